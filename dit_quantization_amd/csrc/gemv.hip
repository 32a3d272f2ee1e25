// W4A16 decode product y = x W^T for NVFP4 weights and bf16 activations,
// M <= 16 rows ("Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de
// laptop", section 2: W4A16 stores 4-bit weights and unpacks them to 16 bits
// for the multiply; decoding reads every weight once per token and is bound
// by memory bandwidth).
//
// M > 1 design (gfx950): a workgroup of NW waves owns 16 * T weight rows;
// its waves split K.  K is read in super-chunks of 128 (4 chunks of 32
// codes = 16 bytes per row), 4 super-chunks per pass.  Lane (n, g) of a wave
// (n = lane % 16, g = lane / 16) takes chunk 4s + g of row n and unpacks its
// 4 code dwords to exact bf16 values q * s_b (<= 6 significant bits,
// magnitudes in [2^-10, 2688]) as the B operands of 4
// v_mfma_f32_16x16x32_bf16.  The codes of a pass reach LDS by DMA with every
// instruction reading 4 rows x 256 contiguous bytes (measured 1.3-2.7 us per
// 33 MB call faster than loading 16 rows x 64 bytes straight into the MFMA
// layout), and each lane reads its chunks back from a row-swizzled slot.  The
// scales of a pass come from one 8-byte load per lane, redistributed between
// the 4 lanes of a row with two cross-lane exchanges.  The loads alone take
// about two thirds of a call; the decode with its per-element block-scale
// multiply and, at M > 4, the x loads take the rest, so the x operand is
// built from as few load instructions as possible:
//  * M <= 4 on weights of fewer than 8192 rows (staggered): lane (4 j + i, g) loads the 8 values of x[i] that
//    meet MFMA j in lane group g -- one 16-byte load per lane covers all 4
//    MFMAs of a super-chunk.  MFMA j keeps only the lanes with j' == j, so
//    output row 4 j + i collects x[i] times the codes of MFMA j, and the
//    4 row blocks are added across lane groups at the end.
//  * otherwise (dense): lane (m, g) holds x[m] on its lane group's k slots for
//    each MFMA; 4 loads per super-chunk cover 16 rows (rows past M read zeros).
// Rows past N, chunks past K and x rows past M are buffer loads at an
// out-of-range offset, which return zero without a memory access.  With the
// dense layout each 16-row tile is computed as soon as its own DMA has
// landed.  Waves are added in LDS in wave order; the epilogue multiplies by
// s_g and rounds to bf16 (RNE).  Workgroups of 16 (or 32 / 64 rows on tall weights) read x
// from L2 once each; M > 4 on short weights with long rows splits K over
// workgroups instead (partial sums added in range order by a second pass).
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

// 8 codes -> 8 exact bf16 values q * sb.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8_scaled(uint32_t c, float sb) {
  float q[8];
  fp4x8_to_f32(c, q);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)(q[j] * sb);
  return r;
}

// Sum of v over the 4 lane groups (lanes n, n+16, n+32, n+48): lane (n, g)
// returns the total of component g.
__device__ __forceinline__ float group_sum4(f32x4 v, int lane) {
  const bool u32 = (lane & 32) != 0, u16 = (lane & 16) != 0;
  float k0 = u32 ? v[2] : v[0], k1 = u32 ? v[3] : v[1];
  float s0 = u32 ? v[0] : v[2], s1 = u32 ? v[1] : v[3];
  k0 += __shfl_xor(s0, 32);
  k1 += __shfl_xor(s1, 32);
  float k = u16 ? k1 : k0, s = u16 ? k0 : k1;
  return k + __shfl_xor(s, 16);
}

// Scale pairs of a pass.  Lane (n, g) loaded the 8 scale bytes of row n for
// super-chunk s0 + g: halfword h = the two block scales of chunk 4 (s0 + g)
// + h.  Returns in pair[u] the two scales of the lane's own chunk
// 4 (s0 + u) + g, for u = 0..3 (a 4 x 4 transpose of halfwords between the
// lanes n, n + 16, n + 32, n + 48).
__device__ __forceinline__ void scale_pairs(u32x2 d, int lane, uint32_t pair[4]) {
  const int g = lane >> 4;
  const bool b1 = (g & 2) != 0, b0 = (g & 1) != 0;
  const uint32_t keep = b1 ? d.y : d.x;  // halfwords b, b+1 (b = g & 2) of super-chunk s0 + g
  const uint32_t recv = __shfl_xor(b1 ? d.x : d.y, 32);  // the same halfwords of super-chunk s0 + (g ^ 2)
  const uint32_t send = b0 ? ((keep & 0xFFFFu) | (recv << 16)) : ((keep >> 16) | (recv & 0xFFFF0000u));
  const uint32_t other = __shfl_xor(send, 16);  // halfword g of super-chunks s0 + (g ^ 1), s0 + (g ^ 3)
  const uint32_t own = b0 ? (keep >> 16) : (keep & 0xFFFFu);
  const uint32_t opp = b0 ? (recv >> 16) : (recv & 0xFFFFu);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d2 = u ^ g;  // 0: own, 2: opp, 1: other.lo, 3: other.hi
    pair[u] = d2 == 0 ? own : d2 == 2 ? opp : d2 == 1 ? (other & 0xFFFFu) : (other >> 16);
  }
}

// s_waitcnt until at most k groups of G vector memory instructions newer
// than the awaited one are outstanding (k < 4; the count must be an
// immediate).
template <int G>
__device__ __forceinline__ void wait_vm_newer(int k) {
  if (k == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  else if (k == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(G));
  else if (k == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * G));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * G));
}

// grid: ceil(N / (16 T)) workgroups of NW waves (times `splits` with
// SPLIT).  DENSE: the M > 4 operand layout; otherwise staggered (M <= 4).
// SPLIT: workgroup b takes super-chunk range b % splits of row block
// b / splits and stores its unscaled fp32 sums in partial [splits, M, N]
// (gemv_splitk_reduce_kernel adds them in range order).
template <int DENSE, int T, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void gemv_w4a16_kernel(const uint16_t* __restrict__ x,
                                                             const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ sg_ptr, int M, int N, int K,
                                                             int bf16_out, void* __restrict__ out, int splits,
                                                             float* __restrict__ partial) {
  constexpr int SW = 4;              // super-chunks per pass (one 8-byte scale load per lane)
  constexpr int XL = DENSE ? 4 : 1;  // x loads per super-chunk
  // Per wave and row tile: the pass's 16 rows x 16 code chunks, staged
  // global -> LDS; the reduction at the end reuses the wave's own region.
  __shared__ u32x4 lds_c[NW][T][256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int split = SPLIT ? (int)(blockIdx.x % splits) : 0;
  const int n0 = (SPLIT ? (int)(blockIdx.x / splits) : (int)blockIdx.x) * (16 * T);
  const int rows = min(16 * T, N - n0);
  const int half = K / 2, sbytes = K / 16;
  const __amdgpu_buffer_rsrc_t cbuf = make_buf(codes + (int64_t)n0 * half, (uint32_t)(rows * half));
  const __amdgpu_buffer_rsrc_t sbuf = make_buf(scales + (int64_t)n0 * sbytes, (uint32_t)(rows * sbytes));
  const __amdgpu_buffer_rsrc_t xbuf = make_buf(x, (uint32_t)(M * K * 2));
  const int nch = K / 32;
  const int nsc = (nch + 3) / 4;
  const int sps = SPLIT ? (nsc + splits - 1) / splits : nsc;  // super-chunks of this workgroup's range
  const int r0 = split * sps, r1 = min(r0 + sps, nsc);
  const int per = (r1 - r0 + NW - 1) / NW;
  const int sbeg = r0 + wave * per, send = min(sbeg + per, r1);
  // x role: dense lane (m, g) holds row m; staggered lane (4 j + i, g) holds
  // row i for MFMA j = jx.
  const int xm = DENSE ? nl : (nl & 3);
  const int jx = nl >> 2;
  auto x_off = [&](int s) {
    const int c = 4 * s + g;
    return (xm < M && s < send && c < nch) ? (xm * K + 32 * c) * 2 + (DENSE ? 0 : 16 * jx) : kBufOOB;
  };

  f32x4 acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool wide_scales = (sbytes & 7) == 0;  // K % 128 == 0: 8-byte aligned scale windows inside each row
  for (int s0 = sbeg; s0 < send; s0 += SW) {  // wave-uniform
    // Issue order: x (L2 hits) for the whole pass, then scales, then codes,
    // so the scale transpose and the first MFMAs wait only for what they use.
    u32x4 xa[SW][XL];
#pragma unroll
    for (int u = 0; u < SW; ++u) {
      const int off = x_off(s0 + u);
#pragma unroll
      for (int j = 0; j < XL; ++j) xa[u][j] = __builtin_amdgcn_raw_buffer_load_b128(xbuf, off + 16 * j, 0, 0);
    }
    // Scale loads are temporal: the waves that split a row's K read
    // neighbouring bytes of the same scale lines (non-temporal, M = 16 took
    // 14.1 / 16.2 us instead of 13.3 / 15.7 us on the two decode shapes).
    u32x2 sw[T];
    {
      // scale bytes [8 (s0 + g), 8 (s0 + g) + 8) of row n
      const int sc = s0 + g;
      const bool ok = sc < send && 4 * sc < nch;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int base = (16 * t + nl) * sbytes + 8 * sc;
        if (wide_scales) {  // uniform
          sw[t] = __builtin_amdgcn_raw_buffer_load_b64(sbuf, ok ? base : kBufOOB, 0, 0);
        } else {            // K % 128 != 0: one halfword per chunk, chunks past K read as zero
          uint32_t h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            h[q] = __builtin_amdgcn_raw_buffer_load_b16(sbuf, ok && 4 * sc + q < nch ? base + 2 * q : kBufOOB, 0, 0);
          sw[t] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        }
      }
    }
    // Codes: DMA instruction u of tile t fills LDS slots [64 u, 64 u + 64):
    // lane l -> row r = 4 u + l / 16, slot j = l % 16, holding chunk
    // 4 s0 + (j ^ r), so each instruction reads 4 rows x 256 contiguous bytes
    // (a permutation of the pass's 16 chunks per row).  Chunks of
    // super-chunks past this wave's range, or past K, read as zero.
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int u = 0; u < SW; ++u) {
        const int r = 4 * u + (lane >> 4);
        const int c = 4 * s0 + ((lane & 15) ^ r);
        const bool ok = c < 4 * send && c < nch;
        // non-temporal: each code byte is read once (decode calls on both
        // shapes 1-5 % faster than with the temporal hint)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(cbuf, (__attribute__((address_space(3))) void*)&lds_c[wave][t][64 * u],
                                                 16, ok ? (16 * t + r) * half + 16 * c : kBufOOB, 0, 0, kBufNT);
      }
    uint32_t pairs[T][4];
    // Lane (n, g) reads chunk 4 (s0 + u) + g of row n from slot (4 u + g) ^ n:
    // the 16 lanes of a group hit 16 different slots of 16 rows (no bank
    // conflicts).
    auto mfma4 = [&](int u, int t, const u32x4& cw) {
      const f32x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(pairs[t][u], 1.0f, false);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        const u32x4 a = DENSE ? xa[u][DENSE ? j : 0] : (jx == j ? xa[u][0] : z4);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         fp4x8_to_bf16x8_scaled(cw[j], j < 2 ? sc.x : sc.y),
                                                         acc[t], 0, 0, 0);
      }
    };
    if constexpr (DENSE) {
#pragma unroll
      for (int t = 0; t < T; ++t) scale_pairs(sw[t], lane, pairs[t]);
      // Tile by tile: tile t's rows come only from its own SW instructions,
      // issued in tile order, so tile t is complete once SW (T - 1 - t)
      // newer loads are outstanding (loads, LDS DMA included, complete in
      // issue order) and its MFMAs overlap the later tiles' DMA.
#pragma unroll
      for (int t = 0; t < T; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_newer<SW>(T - 1 - t);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 cw[SW];
#pragma unroll
        for (int u = 0; u < SW; ++u) cw[u] = lds_c[wave][t][16 * nl + ((4 * u + g) ^ nl)];
#pragma unroll
        for (int u = 0; u < SW; ++u)
          if (s0 + u < send) mfma4(u, t, cw[u]);  // wave-uniform
      }
    } else {
      // Staggered (2-tile workgroups): one wait for the pass, and the tiles'
      // independent accumulators interleaved (faster here: measured).
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
      u32x4 cw[SW][T];
#pragma unroll
      for (int u = 0; u < SW; ++u)
#pragma unroll
        for (int t = 0; t < T; ++t) cw[u][t] = lds_c[wave][t][16 * nl + ((4 * u + g) ^ nl)];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < T; ++t) scale_pairs(sw[t], lane, pairs[t]);
#pragma unroll
      for (int u = 0; u < SW; ++u)
        if (s0 + u < send)  // wave-uniform
#pragma unroll
          for (int t = 0; t < T; ++t) mfma4(u, t, cw[u][t]);
    }
  }

  // dense: lane (n, g) holds rows m = 4 g + i.  staggered: lane (n, g) holds
  // rows 4 g + i = x row i times the codes of MFMA g; the sum over the lane
  // groups leaves row m = g in lane (n, g).
  // (each wave's partial sums go to the first T KB of its own code region)
  f32x4* const red_w = reinterpret_cast<f32x4*>(&lds_c[wave][0][0]);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (DENSE) {
      red_w[64 * t + lane] = acc[t];
    } else {
      const float v = group_sum4(acc[t], lane);
      red_w[64 * t + lane] = f32x4{v, 0.f, 0.f, 0.f};
    }
  }
  __syncthreads();
  const float sg = *sg_ptr;
  for (int idx = threadIdx.x; idx < T * 64; idx += NW * 64) {
    const int t = idx >> 6, l = idx & 63;
    f32x4 sum = reinterpret_cast<const f32x4*>(&lds_c[0][0][0])[64 * t + l];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += reinterpret_cast<const f32x4*>(&lds_c[w][0][0])[64 * t + l];
    const int n = n0 + 16 * t + (l & 15);
#pragma unroll
    for (int i = 0; i < (DENSE ? 4 : 1); ++i) {
      const int m = DENSE ? 4 * (l >> 4) + i : (l >> 4);
      if (m < M && n < N) {
        if (SPLIT)
          partial[((int64_t)split * M + m) * N + n] = sum[i];
        else if (bf16_out)
          reinterpret_cast<uint16_t*>(out)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(sum[i] * sg);
        else
          reinterpret_cast<float*>(out)[(int64_t)m * N + n] = sum[i] * sg;
      }
    }
  }
}

// ---- M = 1: VALU dot products.
// A workgroup (4 waves) owns RW rows per row group; its waves split K into S
// parts and the 4/S row groups split the rows.  Lane l of a wave owns the
// 16-byte code chunks l, l + 64, ... of its K part (chunk c = codes of k in
// [32c, 32c+32)), so one load instruction reads 1 KB of a row contiguously,
// and the lane keeps x for its k's in registers for all of its rows.  Codes
// become bf16 pairs with the hardware converter (scale-free q values, exact);
// v_dot2_f32_bf16 multiplies them with x pairs; each 16-element block sum is
// multiplied by its scale, decoded by the hardware FP8 (E4M3) converter.
// Every load is a buffer load; lanes past the K part (or rows past N) read
// zeros, so their contribution is exactly 0 with no per-lane select.  The
// loads are issued row by row and the rows are computed in the same order
// (scheduling barriers), so a wave starts on its first row while the later
// rows' loads are still in flight.  Rows are reduced across the wave with a
// transposing butterfly, then across the S waves in LDS.
__device__ __forceinline__ void fp4x8_to_bf16x2(uint32_t c, uint32_t v[4]) {
  v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 0));
  v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 1));
  v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 2));
  v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 3));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum v[r] over the 64 lanes for every r < R (R a power of two <= 64).  The
// first log2(R) butterfly steps halve the number of live values per lane:
// afterwards lane l holds row ((l / (64 / R)) bit-reversed order handled by
// the caller through `reduced_row`) partial sums, and the remaining steps
// finish each row.  Result: lane l with (l % (64 / R)) == 0 holds the total
// of row reduced_row(l).
template <int R>
__device__ __forceinline__ float wave_sum_rows(float (&v)[R], int lane) {
  int live = R;
#pragma unroll
  for (int o = 32; o >= 64 / R && live > 1; o >>= 1) {
    const bool upper = (lane & o) != 0;
    const int half = live / 2;
#pragma unroll
    for (int i = 0; i < R / 2; ++i) {
      if (i < half) {
        // lower lanes keep values [0, half), upper lanes keep [half, live)
        float send = upper ? v[i] : v[i + half];
        float keep = upper ? v[i + half] : v[i];
        v[i] = keep + __shfl_xor(send, o);
      }
    }
    live = half;
  }
  float t = v[0];
#pragma unroll
  for (int o = 32 / R; o > 0; o >>= 1) t += __shfl_xor(t, o);
  return t;
}

// Row index held by lane l after wave_sum_rows<R>: bit j of the row number
// is bit (5 - j) of the lane (the butterfly keeps the upper half of the live
// rows in lanes whose bit 5, 4, ... is set).
template <int R>
__device__ __forceinline__ int reduced_row(int lane) {
  int r = 0;
#pragma unroll
  for (int j = 0, o = 32; (1 << j) < R; ++j, o >>= 1) r = 2 * r + ((lane & o) ? 1 : 0);
  return r;
}

template <int CH, int RW, int S>
__global__ __launch_bounds__(256) void gemv_m1_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ sg_ptr, int N, int K, int bf16_out,
                                                      void* __restrict__ out) {
  constexpr int G = 4 / S;                 // row groups per workgroup
  __shared__ float red[4][RW];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave % S, grp = wave / S;
  const int nch = K / 32;
  const int per = (nch + S - 1) / S;       // chunks in each K part
  const int cbeg = part * per, cend = min(cbeg + per, nch);
  const int row0 = (blockIdx.x * G + grp) * RW;
  // this wave's rows (none past N: a row group past the end reads only zeros)
  const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(RW, N - row0)));
  const int64_t rb = min(row0, N - 1);
  const __amdgpu_buffer_rsrc_t cbuf = make_buf(codes + rb * (K / 2), (uint32_t)(nrows * (K / 2)));
  const __amdgpu_buffer_rsrc_t sbuf = make_buf(scales + rb * (K / 16), (uint32_t)(nrows * (K / 16)));
  const __amdgpu_buffer_rsrc_t xbuf = make_buf(x, (uint32_t)(K * 2));
  // x for this lane's chunks (16 dwords = 32 bf16 per chunk)
  uint32_t xr[CH][16];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = cbeg + lane + 64 * c;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xbuf, ch < cend ? 64 * ch + 16 * q : kBufOOB, 0, 0);
      xr[c][4 * q] = v.x; xr[c][4 * q + 1] = v.y; xr[c][4 * q + 2] = v.z; xr[c][4 * q + 3] = v.w;
    }
  }
  u32x4 cw[RW][CH];
  uint32_t sw[RW][CH];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = cbeg + lane + 64 * c;
      cw[r][c] = __builtin_amdgcn_raw_buffer_load_b128(cbuf, ch < cend ? r * (K / 2) + 16 * ch : kBufOOB, 0, kBufNT);
      sw[r][c] = __builtin_amdgcn_raw_buffer_load_b16(sbuf, ch < cend ? r * (K / 16) + 2 * ch : kBufOOB, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);     // issue order = row order
  }
  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    acc[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint32_t q[16];
      fp4x8_to_bf16x2(cw[r][c].x, q);
      fp4x8_to_bf16x2(cw[r][c].y, q + 4);
      fp4x8_to_bf16x2(cw[r][c].z, q + 8);
      fp4x8_to_bf16x2(cw[r][c].w, q + 12);
      float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) p0 = dot2(xr[c][i], q[i], p0);
#pragma unroll
      for (int i = 8; i < 16; ++i) p1 = dot2(xr[c][i], q[i], p1);
      const f32x2 s = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[r][c], 1.0f, false);  // bytes 0, 1 (exact)
      acc[r] = __builtin_fmaf(p1, s[1], __builtin_fmaf(p0, s[0], acc[r]));
    }
    __builtin_amdgcn_sched_barrier(0);     // compute order = row order
  }
  const float tot = wave_sum_rows<RW>(acc, lane);
  if ((lane & (64 / RW - 1)) == 0) red[wave][reduced_row<RW>(lane)] = tot;
  __syncthreads();
  if (threadIdx.x < G * RW) {
    const int g = threadIdx.x / RW, r = threadIdx.x % RW;
    float sum = red[g * S][r];
#pragma unroll
    for (int p = 1; p < S; ++p) sum += red[g * S + p][r];
    const int row = (blockIdx.x * G + g) * RW + r;
    const float sg = *sg_ptr;
    if (row < N) {
      if (bf16_out)
        reinterpret_cast<uint16_t*>(out)[row] = (uint16_t)f32_to_bf16_bits(sum * sg);
      else
        reinterpret_cast<float*>(out)[row] = sum * sg;
    }
  }
}

// y = round(s_g * (((p_0 + p_1) + ...) + p_{S-1})) per element.
__global__ __launch_bounds__(256) void gemv_splitk_reduce_kernel(const float* __restrict__ partial, int splits,
                                                                 int64_t n, const float* __restrict__ sg_ptr,
                                                                 void* __restrict__ y, int bf16_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = partial[i];
  for (int t = 1; t < splits; ++t) s += partial[t * n + i];
  const float v = s * (*sg_ptr);
  if (bf16_out)
    reinterpret_cast<uint16_t*>(y)[i] = (uint16_t)f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(y)[i] = v;
}

int gemv_max_splits(int64_t M, int64_t N) {
  // M > 4 on weights with fewer than 8192 rows: 64-row blocks, about 256
  // workgroups in all (x is read once per workgroup, so the rows per
  // workgroup, not the K range, set its L2 traffic).
  if (M <= 4 || M > 16 || N >= 8192 || N == 0) return 1;
  const int64_t blocks = (N + 63) / 64;
  const int64_t s = (256 + blocks - 1) / blocks;
  return (int)(s > 8 ? 8 : s);
}

int gemv_splits(int64_t M, int64_t N, int64_t K) {
  int s = gemv_max_splits(M, N);
  const int64_t nsc = (K / 32 + 3) / 4;
  if (K < 8192 || s > nsc / 16) s = (int)(K < 8192 ? 1 : nsc / 16);  // long rows only, >= 16 super-chunks a range
  if (s <= 1) return 1;
  const int64_t sps = (nsc + s - 1) / s;
  return (int)((nsc + sps - 1) / sps);
}

hipError_t launch_gemv_w4a16(const uint16_t* x, const uint8_t* codes, const uint8_t* scales, const float* sg,
                             int64_t M, int64_t N, int64_t K, void* y, bool bf16_out, float* partial,
                             hipStream_t stream) {
  int b = bf16_out ? 1 : 0;
  const int64_t nch = K / 32;                      // 16-byte code chunks per row
  if (M == 1 && nch <= 4 * 64 * 4) {
#define NVFP4_GEMV_M1(CH, RW, S)                                                                                  \
  hipLaunchKernelGGL((gemv_m1_kernel<CH, RW, S>), dim3((unsigned)((N + (4 / S) * RW - 1) / ((4 / S) * RW))),      \
                     dim3(256), 0, stream, x, codes, scales, sg, (int)N, (int)K, b, y)
    // 4 rows per wave (8 rows per wave leaves each wave's arithmetic after
    // most of its loads have landed); K in 2 parts up to 16384, else 4.
    if (nch <= 2 * 64) NVFP4_GEMV_M1(1, 4, 2);          // K <= 4096
    else if (nch <= 2 * 128) NVFP4_GEMV_M1(2, 4, 2);    // K <= 8192
    else if (nch <= 2 * 256) NVFP4_GEMV_M1(4, 4, 2);    // K <= 16384
    else NVFP4_GEMV_M1(4, 4, 4);                         // K <= 32768
#undef NVFP4_GEMV_M1
    return hipGetLastError();
  }
  // M > 1: MFMA kernels.  On weights of at least 8192 rows, the dense layout
  // with 64 rows per workgroup of 8 waves for every M (each x fragment feeds
  // 4 row tiles, and x is read from L2 once per workgroup); else 16 rows,
  // with the staggered layout and 8 waves at M <= 4, and the dense layout
  // with 16 waves splitting rows of K >= 8192 at M > 4 (unless the split-K
  // path above took the call).  Chosen by sweeping layout x rows x waves on
  // the 14336 x 4096 and 4096 x 14336 decode shapes (M = 4: 10.7 -> 10.2 and
  // 12.0 -> 11.7 us per call against 32-row staggered tiles and 16 waves).
  const int dense = M > 4 ? 1 : 0;
  const bool t2 = N >= 32 * 256;
  const bool nw16 = !t2 && K >= 8192;
#define NVFP4_GEMV_MFMA(D, T, NW)                                                                                 \
  hipLaunchKernelGGL((gemv_w4a16_kernel<D, T, NW, false>), dim3((unsigned)((N + 16 * T - 1) / (16 * T))),         \
                     dim3(NW * 64), 0, stream, x, codes, scales, sg, (int)M, (int)N, (int)K, b, y, 1, nullptr)
  const int splits = partial ? gemv_splits(M, N, K) : 1;
  if (splits > 1) {
    // 64-row blocks, each split into `splits` K ranges, then the ordered sum.
    hipLaunchKernelGGL((gemv_w4a16_kernel<1, 4, 8, true>), dim3((unsigned)(((N + 63) / 64) * splits)), dim3(512), 0,
                       stream, x, codes, scales, sg, (int)M, (int)N, (int)K, b, y, splits, partial);
    const int64_t n = M * N;
    hipLaunchKernelGGL(gemv_splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, partial,
                       splits, n, sg, y, b);
    return hipGetLastError();
  }
  if (t2) NVFP4_GEMV_MFMA(1, 4, 8);
  else if (!dense) NVFP4_GEMV_MFMA(0, 1, 8);
  else if (nw16) NVFP4_GEMV_MFMA(1, 1, 16);
  else NVFP4_GEMV_MFMA(1, 1, 8);
#undef NVFP4_GEMV_MFMA
  return hipGetLastError();
}

}  // namespace nvfp4
