// W4A16 decode product y = x W^^T for NVFP4 weights and bf16 activations,
// M <= 16 rows ("Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de
// laptop", section 2: W4A16 stores 4-bit weights and unpacks them to 16 bits
// for the multiply; decoding reads every weight once per token and is bound
// by memory bandwidth).
//
// Design (gfx950): one workgroup of 8 waves owns 16 weight rows and all of K.
// K is cut into 32 segments (8 waves x 4 lane groups); lane (n, h) of wave w
// owns segment 4w + h of row n and issues every 16-byte load of its packed
// codes and scales up front, so a workgroup keeps its whole share of the
// weights in flight (about 64 KB per CU), then feeds
// v_mfma_f32_16x16x32_bf16: B = exact bf16 values q * s_b of its codes
// (<= 6 significant bits, magnitudes in [2^-10, 2688]), A = the matching
// x[m, k] (read from L2, double buffered).  Lane groups hold different k
// ranges but A and B use the same k for the same lane, which is all an MFMA
// needs.  The 8 waves' fp32 partial tiles are added in LDS in wave order;
// the fp32 epilogue multiplies by s_g and rounds to bf16 (RNE).  One kernel,
// no workspace.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {
constexpr int kRows = 16;       // weight rows per workgroup (one MFMA tile)
constexpr int kWaves = 8;
constexpr int kSegs = kWaves * 4;
}  // namespace

// Unpack 8 codes (one dword) times the block scale into 8 exact bf16 values.
__device__ __forceinline__ bf16x8 unpack8_bf16(uint32_t c, float sb) {
  float q[8];
  fp4x8_to_f32(c, q);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)(q[j] * sb);
  return r;
}

// grid: ceil(N / 16) workgroups of 512 threads.  Segment length q (a
// multiple of 32) covers K in kSegs segments; TMAX >= q / 32 chunks of 32
// codes per lane are loaded at once (longer segments loop).
// bf16_out: y bf16 [M, N]; otherwise fp32.
template <int TMAX>
__global__ __launch_bounds__(512) void gemv_w4a16_kernel(const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ sg_ptr, int M, int N, int K,
                                                         int q, int bf16_out, void* __restrict__ out) {
  __shared__ f32x4 red[kWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;   // B column (weight row) / A row (x row)
  const int h = lane >> 4;    // lane group
  const int n0 = blockIdx.x * kRows;
  const int row = min(n0 + nl, N - 1);
  const int kseg = (4 * wave + h) * q;
  const int kend = min(kseg + q, K);
  const uint8_t* crow = codes + (int64_t)row * (K / 2);
  const uint8_t* srow = scales + (int64_t)row * (K / 16);
  const bool a_live = nl < M;
  const uint16_t* xrow = x + (int64_t)(a_live ? nl : 0) * K;

  // Every lane runs the same passes and MFMAs (an MFMA reads the operand
  // registers of all 64 lanes); chunks outside a lane's segment are zero.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < q; p0 += 32 * TMAX) {
    const int kp = kseg + p0;
    // all weight loads of this pass first
    u32x4 cw[TMAX];
    uint32_t sw[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      int k = kp + 32 * t;
      int kk = k < kend ? k : 0;
      cw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + kk / 2));
      sw[t] = *reinterpret_cast<const uint16_t*>(srow + kk / 16);
    }
    // x for the first chunk: unconditional loads from a clamped k.  A rows
    // m >= M only reach output rows that are never stored, and chunks past a
    // segment meet zero B operands, so these values need no masking.
    u32x4 xa[2][4];
    {
      const int kc = kp < kend ? kp : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[0][j] = *reinterpret_cast<const u32x4*>(xrow + kc + 8 * j);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int k = kp + 32 * t;
      const bool live = k < kend;
      const int cur = t & 1;
      if (t + 1 < TMAX) {
        const int k1 = k + 32;
        const int kc = k1 < kend ? k1 : 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[cur ^ 1][j] = *reinterpret_cast<const u32x4*>(xrow + kc + 8 * j);
      }
      const float sb0 = e4m3_to_f32(sw[t] & 0xFFu), sb1 = e4m3_to_f32(sw[t] >> 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b = live ? unpack8_bf16(cw[t][j], j < 2 ? sb0 : sb1) : bf16x8{};
        bf16x8 a = __builtin_bit_cast(bf16x8, xa[cur][j]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
      }
    }
  }

  // acc[i] = partial C[m = 4h + i][n = nl]; add the 8 waves in order.
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 s = red[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[w][lane];
    const float sg = *sg_ptr;
    const int n = n0 + nl;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * h + i;
        if (m >= M) continue;
        if (bf16_out)
          reinterpret_cast<uint16_t*>(out)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(s[i] * sg);
        else
          reinterpret_cast<float*>(out)[(int64_t)m * N + n] = s[i] * sg;
      }
    }
  }
}

// ---- M = 1: VALU dot products.
// A workgroup (4 waves) owns RW rows; its waves split K into S parts and the
// 4/S row groups split the rows.  Lane l of a wave owns the 16-byte code
// chunks l, l + 64, ... of its K part (chunk c = codes of k in [32c, 32c+32)),
// so one load instruction reads 1 KB of a row contiguously, and the lane
// keeps x for its k's in registers for all of its rows.  Codes become bf16
// pairs with the hardware converter (scale-free q values, exact);
// v_dot2_f32_bf16 multiplies them with x pairs; each 16-element block sum is
// multiplied by its scale.  Rows are reduced across the wave with a
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = wave % S, grp = wave / S;
  const int nch = K / 32;
  const int per = (nch + S - 1) / S;       // chunks in each K part
  const int cbeg = part * per, cend = min(cbeg + per, nch);
  const int row0 = (blockIdx.x * G + grp) * RW;
  // x for this lane's chunks (16 dwords = 32 bf16 per chunk), clamped past the part
  uint32_t xr[CH][16];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = min(cbeg + lane + 64 * c, nch - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 v = *reinterpret_cast<const u32x4*>(x + 32 * ch + 8 * q);
      xr[c][4 * q] = v.x; xr[c][4 * q + 1] = v.y; xr[c][4 * q + 2] = v.z; xr[c][4 * q + 3] = v.w;
    }
  }
  // all weight loads of this wave first
  u32x4 cw[RW][CH];
  uint32_t sw[RW][CH];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = min(row0 + r, N - 1);
    const uint8_t* crow = codes + (int64_t)row * (K / 2);
    const uint8_t* srow = scales + (int64_t)row * (K / 16);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = min(cbeg + lane + 64 * c, nch - 1);
      cw[r][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + 16 * ch));
      sw[r][c] = *reinterpret_cast<const uint16_t*>(srow + 2 * ch);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    acc[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const bool live = cbeg + lane + 64 * c < cend;
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
      const float s0 = e4m3_to_f32(sw[r][c] & 0xFFu), s1 = e4m3_to_f32(sw[r][c] >> 8);
      acc[r] = live ? __builtin_fmaf(p1, s1, __builtin_fmaf(p0, s0, acc[r])) : acc[r];
    }
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

hipError_t launch_gemv_w4a16(const uint16_t* x, const uint8_t* codes, const uint8_t* scales, const float* sg,
                             int64_t M, int64_t N, int64_t K, void* y, bool bf16_out, hipStream_t stream) {
  int b = bf16_out ? 1 : 0;
  const int64_t nch = K / 32;                      // 16-byte code chunks per row
  if (M == 1 && nch <= 4 * 64 * 4) {
#define NVFP4_GEMV_M1(CH, RW, S)                                                                                  \
  hipLaunchKernelGGL((gemv_m1_kernel<CH, RW, S>), dim3((unsigned)((N + (4 / S) * RW - 1) / ((4 / S) * RW))),      \
                     dim3(256), 0, stream, x, codes, scales, sg, (int)N, (int)K, b, y)
    if (nch <= 2 * 64) NVFP4_GEMV_M1(1, 8, 2);          // K <= 4096: halves of the row per wave
    else if (nch <= 4 * 128) NVFP4_GEMV_M1(2, 8, 4);    // K <= 16384: quarters
    else NVFP4_GEMV_M1(4, 4, 4);                         // K <= 32768
#undef NVFP4_GEMV_M1
    return hipGetLastError();
  }
  int64_t q = ((K + kSegs - 1) / kSegs + 31) / 32 * 32;   // segment length, a multiple of 32
  int64_t chunks = q / 32;
  dim3 grid((unsigned)((N + kRows - 1) / kRows));
  if (chunks <= 4)
    hipLaunchKernelGGL(gemv_w4a16_kernel<4>, grid, dim3(512), 0, stream, x, codes, scales, sg, (int)M, (int)N,
                       (int)K, (int)q, b, y);
  else if (chunks <= 8)
    hipLaunchKernelGGL(gemv_w4a16_kernel<8>, grid, dim3(512), 0, stream, x, codes, scales, sg, (int)M, (int)N,
                       (int)K, (int)q, b, y);
  else
    hipLaunchKernelGGL(gemv_w4a16_kernel<16>, grid, dim3(512), 0, stream, x, codes, scales, sg, (int)M, (int)N,
                       (int)K, (int)q, b, y);
  return hipGetLastError();
}

}  // namespace nvfp4
