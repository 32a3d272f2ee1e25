// Per-call NVFP4 quantization of the W4A4 product's bf16 activation for
// gfx950, alone or fused with the down projection of a low-rank branch.
//
// "NVFP4 en difusion: la misma cuantizacion, un motor completamente
// distinto", section 2 ("NVFP4 sin vLLM: torch._scaled_mm a mano"): the
// activation is quantized to NVFP4 on every call, 16-element block by block,
// with the same absmax criterion as the weights; section 3: a LoRA (or
// SVDQuant's low-rank part) runs in the same pass, in 16 bits.
//
// Output: the exact fp16 values q_a * s_a (<= 6 significant bits,
// magnitudes in [2^-10, 2688]) that the product's fp16 matrix cores read,
// and s_gA in the workspace.  The tensor scale comes from this call's amax
// partials, reduced by every workgroup of the pass itself (no separate
// finalize launch), or from the caller.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------- act quant

// The pass's tensor scale (see ActScale): the given value, or fp32(amax /
// 2688) from the amax partials of this call (at most kMaxAmaxPartials,
// 256 threads: every partial is requested before any is used).  Max is exact
// and order-free, so every workgroup gets the same value, equal to what a
// separate reduction pass would produce.  Called by all 256 threads.
__device__ __forceinline__ float act_scale_256(const ActScale& s) {
  constexpr int kLoads = (kMaxAmaxPartials + 255) / 256;  // every partial requested in one batch
  __shared__ float red[4];
  float sg;
  if (s.partials == nullptr) {
    sg = *s.src;
  } else {
    float v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int i = threadIdx.x + 256 * j;
      v[j] = i < s.np ? s.partials[i] : 0.0f;
    }
    float m = v[0];
#pragma unroll
    for (int j = 1; j < kLoads; ++j) m = fmaxf(m, v[j]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    sg = global_scale_from_amax(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *s.out = sg;
  return sg;
}

// 8 bf16 values (half a block; the other half is in lane l ^ 1) -> their
// quantized values q * s_b as fp16 (exact).
__device__ __forceinline__ u32x4 act_quant_half(u32x4 v, float sg, float inv_sg, double six_sg) {
  float w[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[2 * j] = bf16_bits_to_f32(v[j] & 0xFFFFu);
    w[2 * j + 1] = bf16_bits_to_f32(v[j] >> 16);
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(w[j]));
  m = fmaxf(m, __shfl_xor(m, 1));
  uint32_t sc = e4m3_code_rne((double)m / six_sg);
  float sb = e4m3_to_f32(sc);
  uint32_t codes = encode8(w, sb, sg, inv_sg);
  _Float16 sbh = (_Float16)sb;
  f16x2 s2 = {sbh, sbh};
  f16x2 q[4];
  fp4x8_to_f16x2(codes, q);
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = __builtin_bit_cast(uint32_t, q[j] * s2);
  return o;
}

// One lane per half block of the bf16 activation; lanes 2b, 2b+1 share block
// b.  Each lane takes two half blocks a grid stride apart per iteration and
// issues both loads before using either (plain loads: the activation was
// usually just written or read by the amax pass and may still be cached).
// Measured 8-11 % faster than one half block per iteration with
// non-temporal loads on the prefill and DiT activations.
__global__ __launch_bounds__(256) void act_quant_f16_kernel(const u32x4* __restrict__ a, int64_t n_half,
                                                            ActScale sgs, u32x4* __restrict__ a_hat) {
  const float sg = act_scale_256(sgs);
  const float inv_sg = 1.0f / sg;
  const double six_sg = 6.0 * (double)sg;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; h < n_half; h += 2 * stride) {
    // n_half is even, so lanes 2b and 2b+1 agree on whether h + stride is in range
    const int64_t h1 = h + stride;
    const bool two = h1 < n_half;
    const u32x4 v0 = a[h];
    const u32x4 v1 = two ? a[h1] : u32x4{0u, 0u, 0u, 0u};
    a_hat[h] = act_quant_half(v0, sg, inv_sg, six_sg);
    if (two) a_hat[h1] = act_quant_half(v1, sg, inv_sg, six_sg);
  }
}

hipError_t launch_act_quant_f16(const uint16_t* a, int64_t n_elems, ActScale sg, uint16_t* a_hat,
                                hipStream_t stream) {
  int64_t n_half = n_elems / 8;
  if (n_half == 0) return hipSuccess;  // (M = 0 or K = 0 never reach here: the C ABI returns first)
  // two half blocks per lane; at most 2048 workgroups, each of which reduces
  // the amax partials first (8192 workgroups measured 1-3 us slower on the
  // prefill and DiT activations, interleaved runs)
  int64_t wg = (n_half + 511) / 512;
  if (wg > 2048) wg = 2048;
  hipLaunchKernelGGL(act_quant_f16_kernel, dim3((unsigned)wg), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(a), n_half, sg, reinterpret_cast<u32x4*>(a_hat));
  return hipGetLastError();
}

// Activation quantization fused with the down projection of a low-rank
// (LoRA) branch ("NVFP4 en difusion ...", section 3: the layer computes
// W_4bit x + B (A x), the low-rank term in 16 bits, inside the pass that
// quantizes the activation so x is read once).
//
// A workgroup owns 16 rows and one of `splits` equal ranges of 32-wide K
// chunks (splits > 1 only when there are too few 16-row tiles to fill the
// chip); its 4 waves take the range's chunks round-robin, U chunks per
// batch with every load of the batch in flight before any use.  Lane
// (row, g) loads the 8 bf16 values x[row][32c + 8g, +8): half of a
// 16-element block (lanes g and g^1 share it), quantized exactly as
// act_quant_f16_kernel does, and also the A operand of
// v_mfma_f32_16x16x32_bf16 against lora_down (B operand: lane (j, g) holds
// lora_down[j][32c + 8g, +8)).  Chunks past the range load as zero and add
// nothing.  The 4 waves' fp32 sums are added in LDS in wave order; with one
// split the result is stored as bf16 (RNE) L [M, 16 RT], otherwise as fp32
// partial sums [splits, M, 16 RT] that lora_reduce_kernel adds in split
// order.
//
// SMOOTH (SVDQuant, same section: outliers moved from the activation into
// the weights channel by channel): every loaded x chunk is first replaced by
// bf16(x_k mult_k) with the per-channel fp32 multipliers, and both the
// quantizer and the down projection see that smoothed activation.
template <int RT, bool SMOOTH>
__global__ __launch_bounds__(256) void act_quant_lora_kernel(const uint16_t* __restrict__ a, ActScale sgs,
                                                             const uint16_t* __restrict__ down, int M, int K,
                                                             int splits, int cps, const float* __restrict__ mult,
                                                             uint16_t* __restrict__ a_hat,
                                                             uint16_t* __restrict__ lora_l,
                                                             float* __restrict__ partial) {
  constexpr int R = 16 * RT;
  constexpr int U = RT <= 3 ? 4 : 2;
  __shared__ f32x4 red[4][RT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x / splits, split = blockIdx.x % splits;
  const int m0 = tile * 16;
  const int rows = min(16, M - m0);
  const float sg = act_scale_256(sgs);
  const float inv_sg = 1.0f / sg;
  const double six_sg = 6.0 * (double)sg;
  const __amdgpu_buffer_rsrc_t abuf = make_buf(a + (int64_t)m0 * K, (uint32_t)(rows * K * 2));
  const __amdgpu_buffer_rsrc_t dbuf = make_buf(down, (uint32_t)(R * K * 2));
  const __amdgpu_buffer_rsrc_t mbuf = make_buf(mult, SMOOTH ? (uint32_t)(K * 4) : 0u);
  const int nch = K / 32;
  const int cbeg = split * cps, cend = min(cbeg + cps, nch);
  f32x4 acc[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = cbeg + wave; c0 < cend; c0 += 4 * U) {  // wave-uniform
    u32x4 v[U], d[U][RT], sm[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
      const int k = 32 * c + 8 * g;
      // plain load: the amax pass just read x, and part of it may still be cached
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(abuf, c < cend ? (row * K + k) * 2 : kBufOOB, 0, 0);
      if constexpr (SMOOTH) {
        sm[u][0] = __builtin_amdgcn_raw_buffer_load_b128(mbuf, c < cend ? k * 4 : kBufOOB, 0, 0);
        sm[u][1] = __builtin_amdgcn_raw_buffer_load_b128(mbuf, c < cend ? k * 4 + 16 : kBufOOB, 0, 0);
      }
#pragma unroll
      for (int jt = 0; jt < RT; ++jt)
        d[u][jt] = __builtin_amdgcn_raw_buffer_load_b128(dbuf, c < cend ? ((16 * jt + row) * K + k) * 2 : kBufOOB,
                                                         0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
      const int k = 32 * c + 8 * g;
      if constexpr (SMOOTH)
        v[u] = smooth8(v[u], __builtin_bit_cast(f32x4, sm[u][0]), __builtin_bit_cast(f32x4, sm[u][1]));
      float w[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[2 * j] = bf16_bits_to_f32(v[u][j] & 0xFFFFu);
        w[2 * j + 1] = bf16_bits_to_f32(v[u][j] >> 16);
      }
      float mx = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(w[j]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      const uint32_t sc = e4m3_code_rne((double)mx / six_sg);
      const float sb = e4m3_to_f32(sc);
      const uint32_t codes = encode8(w, sb, sg, inv_sg);
      const _Float16 sbh = (_Float16)sb;
      const f16x2 s2 = {sbh, sbh};
      f16x2 q[4];
      fp4x8_to_f16x2(codes, q);
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = __builtin_bit_cast(uint32_t, q[j] * s2);
      if (row < rows && c < cend) *reinterpret_cast<u32x4*>(a_hat + (int64_t)(m0 + row) * K + k) = o;
#pragma unroll
      for (int jt = 0; jt < RT; ++jt)
        acc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v[u]),
                                                          __builtin_bit_cast(bf16x8, d[u][jt]), acc[jt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) red[wave][jt][lane] = acc[jt];
  __syncthreads();
  if (wave == 0) {
    // lane (j, g) holds L[rows 4g .. 4g+3][16 jt + j]
#pragma unroll
    for (int jt = 0; jt < RT; ++jt) {
      const f32x4 sum = ((red[0][jt][lane] + red[1][jt][lane]) + red[2][jt][lane]) + red[3][jt][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m >= rows) continue;
        const int64_t at = (int64_t)(m0 + m) * R + 16 * jt + row;
        if (splits == 1) lora_l[at] = (uint16_t)f32_to_bf16_bits(sum[i]);
        else partial[(int64_t)split * M * R + at] = sum[i];
      }
    }
  }
}

// L[i] = bf16(((p[0][i] + p[1][i]) + ...) + p[splits-1][i]) over the n = M R
// entries of the split partial sums.
__global__ __launch_bounds__(256) void lora_reduce_kernel(const float* __restrict__ partial, int splits, int64_t n,
                                                          uint16_t* __restrict__ lora_l) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = partial[i];
  for (int t = 1; t < splits; ++t) s += partial[t * n + i];
  lora_l[i] = (uint16_t)f32_to_bf16_bits(s);
}

int lora_splits(int64_t M, int64_t K) {
  // Enough (16-row tile, K range) workgroups to give each CU about four,
  // with at least four chunks (one per wave) in each range.
  const int64_t tiles = (M + 15) / 16, nch = K / 32;
  if (tiles == 0 || tiles >= 1024) return 1;
  int64_t s = (1024 + tiles - 1) / tiles;
  if (s > nch / 4) s = nch / 4;
  if (s <= 1) return 1;
  const int64_t cps = (nch + s - 1) / s;
  return (int)((nch + cps - 1) / cps);  // no empty range
}

hipError_t launch_act_quant_lora(const uint16_t* a, ActScale sg, const uint16_t* down, int rank, int64_t M,
                                 int64_t K, const float* mult, uint16_t* a_hat, uint16_t* lora_l, float* partial,
                                 hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int splits = lora_splits(M, K);
  const int nch = (int)(K / 32);
  const int cps = (nch + splits - 1) / splits;
  const dim3 grid((unsigned)(((M + 15) / 16) * splits));
#define NVFP4_AQL(RT)                                                                                         \
  if (mult)                                                                                                   \
    hipLaunchKernelGGL((act_quant_lora_kernel<RT, true>), grid, dim3(256), 0, stream, a, sg, down, (int)M,    \
                       (int)K, splits, cps, mult, a_hat, lora_l, partial);                                    \
  else                                                                                                        \
    hipLaunchKernelGGL((act_quant_lora_kernel<RT, false>), grid, dim3(256), 0, stream, a, sg, down, (int)M,   \
                       (int)K, splits, cps, mult, a_hat, lora_l, partial)
  switch (rank / 16) {
    case 1: NVFP4_AQL(1); break;
    case 2: NVFP4_AQL(2); break;
    case 3: NVFP4_AQL(3); break;
    case 4: NVFP4_AQL(4); break;
    case 5: NVFP4_AQL(5); break;
    case 6: NVFP4_AQL(6); break;
    case 7: NVFP4_AQL(7); break;
    default: NVFP4_AQL(8); break;
  }
#undef NVFP4_AQL
  if (splits > 1) {
    const int64_t n = M * rank;
    hipLaunchKernelGGL(lora_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, partial, splits,
                       n, lora_l);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
