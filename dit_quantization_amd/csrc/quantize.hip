// NVFP4 quantizer kernels for gfx950: tensor amax -> s_g, and the absmax
// block quantizer.
//
// "Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de laptop", section 2:
// absmax places the block's largest magnitude on the top grid value
// (s = max|W_k| / 6), each element is the nearest grid value of W/(s_b s_g),
// and a per-tensor fp32 scale covers the tensor's range so the 8-bit block
// scale only needs the block's range relative to it.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------- amax

// max |x| over the 8 bf16 or 4 fp32 values of a 16-byte vector.
template <bool kBF16>
__device__ __forceinline__ float absmax16(u32x4 v) {
  float m = 0.0f;
  if constexpr (kBF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, fabsf(bf16_bits_to_f32(v[j] & 0xFFFFu)));
      m = fmaxf(m, fabsf(bf16_bits_to_f32(v[j] >> 16)));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(__uint_as_float(v[j])));
  }
  return m;
}

// Each workgroup reduces a grid-strided share of the tensor (16-byte loads,
// four in flight per lane) to one partial max |x|.  Plain loads: the
// quantizing pass that follows reads the same tensor and may still find part
// of it cached (non-temporal loads here measured 2-4 % slower on the DiT
// block and the dynamic-scale quantize).
template <bool kBF16>
__global__ __launch_bounds__(256) void amax_partial_kernel(const void* __restrict__ x, int64_t n_vec,
                                                           float* __restrict__ partials) {
  float m = 0.0f;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const u32x4 v0 = xv[i], v1 = xv[i + stride], v2 = xv[i + 2 * stride], v3 = xv[i + 3 * stride];
    m = fmaxf(m, fmaxf(fmaxf(absmax16<kBF16>(v0), absmax16<kBF16>(v1)),
                       fmaxf(absmax16<kBF16>(v2), absmax16<kBF16>(v3))));
  }
  for (; i < n_vec; i += stride) m = fmaxf(m, absmax16<kBF16>(xv[i]));
  __shared__ float red[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// The same over the SVDQuant-smoothed bf16 activation bf16(x_k m_k) of a
// row-major [rows, K] tensor (K % 8 == 0): rounding is monotonic, so the
// largest smoothed magnitude is the smoothed value of the largest |x m|.
// Two vectors in flight per lane (each also loads its 8 multipliers).
// Plain loads here too (the SVDQuant DiT block 1.05-1.07 -> 1.04 ms against
// non-temporal ones).
__device__ __forceinline__ float absmax_smooth16(u32x4 v, const f32x4* __restrict__ mult, int kv) {
  return absmax16<true>(smooth8(v, mult[2 * kv], mult[2 * kv + 1]));
}

__global__ __launch_bounds__(256) void amax_smooth_partial_kernel(const u32x4* __restrict__ x, int64_t n_vec,
                                                                  const f32x4* __restrict__ mult, int kvec,
                                                                  float* __restrict__ partials) {
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + stride < n_vec; i += 2 * stride) {
    const u32x4 v0 = x[i], v1 = x[i + stride];
    m = fmaxf(m, fmaxf(absmax_smooth16(v0, mult, (int)(i % kvec)), absmax_smooth16(v1, mult, (int)((i + stride) % kvec))));
  }
  if (i < n_vec) m = fmaxf(m, absmax_smooth16(x[i], mult, (int)(i % kvec)));
  __shared__ float red[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Per-channel running range of a row-major [rows, cols] tensor (cols % 8 ==
// 0): amax[k] = max(amax[k], max_r |x[r][k]|).  A thread owns 8 consecutive
// columns of a stripe of rows; the column maxima meet through unsigned
// atomic max on the float bits (exact and order-free for non-negative
// floats).
template <bool kBF16>
__global__ __launch_bounds__(256) void channel_amax_kernel(const void* __restrict__ x, int64_t rows, int cols,
                                                           float* __restrict__ amax) {
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c0 >= cols) return;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    if constexpr (kBF16) {
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + r * cols + c0));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m[2 * j] = fmaxf(m[2 * j], fabsf(bf16_bits_to_f32(v[j] & 0xFFFFu)));
        m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf(bf16_bits_to_f32(v[j] >> 16)));
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(x) + r * cols + c0) + h);
#pragma unroll
        for (int j = 0; j < 4; ++j) m[4 * h + j] = fmaxf(m[4 * h + j], fabsf(__uint_as_float(v[j])));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) atomicMax(reinterpret_cast<unsigned int*>(amax) + c0 + j, __float_as_uint(m[j]));
}

hipError_t launch_channel_amax(const void* x, bool bf16, int64_t rows, int64_t cols, float* amax,
                               hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const unsigned gx = (unsigned)((cols / 8 + 255) / 256);
  int64_t gy = (1024 + gx - 1) / gx;
  if (gy > rows) gy = rows;
  const dim3 grid(gx, (unsigned)gy);
  if (bf16)
    hipLaunchKernelGGL(channel_amax_kernel<true>, grid, dim3(256), 0, stream, x, rows, (int)cols, amax);
  else
    hipLaunchKernelGGL(channel_amax_kernel<false>, grid, dim3(256), 0, stream, x, rows, (int)cols, amax);
  return hipGetLastError();
}

// kRunningMax: out = max(out, amax) (a running calibration range) instead of
// out = s_g(amax).
template <bool kRunningMax>
__global__ __launch_bounds__(256) void amax_finalize_kernel(const float* __restrict__ partials, int np,
                                                            float* __restrict__ out) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < np; i += blockDim.x) m = fmaxf(m, partials[i]);
  __shared__ float red[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    *out = kRunningMax ? fmaxf(*out, amax) : global_scale_from_amax(amax);
  }
}

int amax_partial_count(int64_t n_elems, bool bf16) {
  int64_t n_vec = n_elems / (bf16 ? 8 : 4);
  int64_t wg = (n_vec + 256 * 4 - 1) / (256 * 4);  // ~4 vectors per thread (one batch of loads)
  if (wg < 1) wg = 1;
  if (wg > kMaxAmaxPartials) wg = kMaxAmaxPartials;
  return (int)wg;
}

static void launch_amax_partials(const void* x, bool bf16, int64_t n_elems, float* partials, int np,
                                 hipStream_t stream) {
  int64_t n_vec = n_elems / (bf16 ? 8 : 4);
  if (bf16)
    hipLaunchKernelGGL(amax_partial_kernel<true>, dim3(np), dim3(256), 0, stream, x, n_vec, partials);
  else
    hipLaunchKernelGGL(amax_partial_kernel<false>, dim3(np), dim3(256), 0, stream, x, n_vec, partials);
}

hipError_t launch_global_scale(const void* x, bool bf16, int64_t n_elems, float* partials, float* sg_out,
                               hipStream_t stream) {
  int np = amax_partial_count(n_elems, bf16);
  launch_amax_partials(x, bf16, n_elems, partials, np, stream);
  hipLaunchKernelGGL(amax_finalize_kernel<false>, dim3(1), dim3(256), 0, stream, partials, np, sg_out);
  return hipGetLastError();
}

hipError_t launch_amax_partials_only(const void* x, bool bf16, int64_t n_elems, float* partials, hipStream_t stream) {
  launch_amax_partials(x, bf16, n_elems, partials, amax_partial_count(n_elems, bf16), stream);
  return hipGetLastError();
}

hipError_t launch_amax_smooth_partials_only(const uint16_t* x, int64_t rows, int64_t K, const float* mult,
                                            float* partials, hipStream_t stream) {
  int np = amax_partial_count(rows * K, true);
  hipLaunchKernelGGL(amax_smooth_partial_kernel, dim3(np), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(x),
                     rows * K / 8, reinterpret_cast<const f32x4*>(mult), (int)(K / 8), partials);
  return hipGetLastError();
}

hipError_t launch_global_scale_smooth(const uint16_t* x, int64_t rows, int64_t K, const float* mult,
                                      float* partials, float* sg_out, hipStream_t stream) {
  int np = amax_partial_count(rows * K, true);
  hipLaunchKernelGGL(amax_smooth_partial_kernel, dim3(np), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(x),
                     rows * K / 8, reinterpret_cast<const f32x4*>(mult), (int)(K / 8), partials);
  hipLaunchKernelGGL(amax_finalize_kernel<false>, dim3(1), dim3(256), 0, stream, partials, np, sg_out);
  return hipGetLastError();
}

hipError_t launch_running_amax(const void* x, bool bf16, int64_t n_elems, float* partials, float* amax,
                               hipStream_t stream) {
  int np = amax_partial_count(n_elems, bf16);
  launch_amax_partials(x, bf16, n_elems, partials, np, stream);
  hipLaunchKernelGGL(amax_finalize_kernel<true>, dim3(1), dim3(256), 0, stream, partials, np, amax);
  return hipGetLastError();
}

// ---------------------------------------------------------------- absmax quantizer

// Grid cap of the absmax pass: 32768 workgroups of 256
// lanes, one half block per lane for tensors up to 67 M elements (a
// 14336 x 4096 weight then runs in a single iteration).  With a cap of 8192
// (3.5 iterations a lane on that weight) the 8B layer set's absmax pass took
// 184-190 us instead of 172-176.
constexpr int64_t kQuantizeMaxGrid = 32768;

// The raw bytes of half block h (elements [8h, 8h+8)): 16 bytes of bf16 or
// 32 of fp32, plain loads (measured 5 % faster than non-temporal ones on
// this pass), unpacked to fp32 once the next half block's loads are issued.
struct Half8 {
  u32x4 a, b;
};

template <bool kBF16>
__device__ __forceinline__ Half8 load_half8(const void* __restrict__ x, int64_t h) {
  Half8 r;
  if constexpr (kBF16) {
    r.a = reinterpret_cast<const u32x4*>(x)[h];
    r.b = u32x4{0u, 0u, 0u, 0u};
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(x) + 2 * h;
    r.a = p[0];
    r.b = p[1];
  }
  return r;
}

template <bool kBF16>
__device__ __forceinline__ void unpack_half8(const Half8& v, float w[8]) {
  if constexpr (kBF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[2 * j] = bf16_bits_to_f32(v.a[j] & 0xFFFFu);
      w[2 * j + 1] = bf16_bits_to_f32(v.a[j] >> 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = __uint_as_float(v.a[j]);
      w[4 + j] = __uint_as_float(v.b[j]);
    }
  }
}

// One lane per half block (8 elements); lanes 2b and 2b+1 share block b.
// x: flat [n] elements (rows*cols, cols % 16 == 0 so blocks never straddle
// rows); codes: 4 bytes per lane; scales: one byte per block, gathered four
// at a time into lane 8q's dword store when `scales` is 4-byte aligned.
template <bool kBF16>
__global__ __launch_bounds__(256) void quantize_absmax_kernel(const void* __restrict__ x, int64_t n_half,
                                                              const float* __restrict__ sg_ptr,
                                                              uint32_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  // A lane's first half block is requested before anything else, and each
  // iteration requests the next one before its own arithmetic (on the 8B
  // layer set in fp32, with a grid of one half block per lane for most
  // tensors: 196 -> 172-176 us).
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;  // a multiple of 64
  int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  Half8 next{};
  if (h < n_half) next = load_half8<kBF16>(x, h);
  const float sg = *sg_ptr;
  const float inv_sg = 1.0f / sg;
  const double six_sg = 6.0 * (double)sg;
  const bool pack = (reinterpret_cast<uintptr_t>(scales) & 3) == 0;
  for (; h < n_half; h += stride) {
    const Half8 cur = next;
    if (h + stride < n_half) next = load_half8<kBF16>(x, h + stride);
    float w[8];
    unpack_half8<kBF16>(cur, w);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(w[j]));
    m = fmaxf(m, __shfl_xor(m, 1));
    uint32_t sc = e4m3_code_rne((double)m / six_sg);
    float sb = e4m3_to_f32(sc);
    __builtin_nontemporal_store(encode8(w, sb, sg, inv_sg), &codes[h]);
    // blocks 4q .. 4q+3 sit in lanes 8q, 8q+2, 8q+4, 8q+6 (h = 8q + lane offset)
    const uint32_t s1 = __shfl_down(sc, 2), s2 = __shfl_down(sc, 4), s3 = __shfl_down(sc, 6);
    if (pack && (h | 7) < n_half) {  // the whole group of 8 lanes is in range (same test in all 8)
      if ((h & 7) == 0) reinterpret_cast<uint32_t*>(scales)[h >> 3] = sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
    } else if ((h & 1) == 0) {
      scales[h >> 1] = (uint8_t)sc;
    }
  }
}

// Four-over-six block scales ("Tu pipeline NVFP4 ...", section 2, algorithm
// table: each block chooses 6 or 4 as the value its maximum maps to, by
// reconstruction error), in the absmax pass's layout: one lane per half
// block, lanes 2b and 2b+1 share block b, so every load is coalesced.  The
// two candidates are the nearest E4M3 values to max / (6 s_g) (the absmax
// scale) and max / (4 s_g).  A candidate's error is
// E = ((d_0^2 + d_1^2) + ...) + d_15^2 in fp64 with d_e = |W_e| - c s_g |q_e|
// rounded once: the even lane sums its 8 terms, the odd lane continues that
// sum with its own 8 in element order, and picks the max -> 4 scale only on a
// strictly smaller error.
template <bool kBF16>
__global__ __launch_bounds__(256) void quantize_4o6_kernel(const void* __restrict__ x, int64_t n_half,
                                                           const float* __restrict__ sg_ptr,
                                                           uint32_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const float sg = *sg_ptr;
  const float inv_sg = 1.0f / sg;
  const double sg64 = (double)sg;
  const bool pack = (reinterpret_cast<uintptr_t>(scales) & 3) == 0;
  const bool odd = (threadIdx.x & 1) != 0;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;  // a multiple of 64
  for (int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; h < n_half; h += stride) {
    // (no load-ahead here: holding the next half block cost this
    // register-heavy pass 2 % on the 8B layer set)
    float w[8];
    unpack_half8<kBF16>(load_half8<kBF16>(x, h), w);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(w[j]));
    m = fmaxf(m, __shfl_xor(m, 1));
    // the even lane rounds max|W| / (6 s_g), the odd lane max|W| / (4 s_g); they swap
    const uint32_t kk = e4m3_code_rne((double)m / ((odd ? 4.0 : 6.0) * sg64));
    const uint32_t ko = (uint32_t)__shfl_xor((int)kk, 1);
    const uint32_t k6 = odd ? ko : kk, k4 = odd ? kk : ko;  // k4 >= k6
    const float c6 = e4m3_to_f32(k6), c4 = e4m3_to_f32(k4);
    const uint32_t word6 = encode8(w, c6, sg, inv_sg);
    uint32_t word = word6, sc = k6;
    if (k4 != k6) {  // the lane pair agrees (same m)
      const uint32_t word4 = encode8(w, c4, sg, inv_sg);
      const double cs6 = (double)c6 * sg64, cs4 = (double)c4 * sg64;  // exact
      float q6[8], q4[8];
      fp4x8_to_f32(word6, q6);
      fp4x8_to_f32(word4, q4);
      // Every lane squares its 8 errors per candidate (d = |w| - c s_g |q|,
      // one rounding: the product is exact).  Only the sums are ordered: the
      // even lane adds terms 0..7 from zero, the odd lane continues from the
      // even lane's sums with terms 8..15, so each E keeps element order.
      double sq6[8], sq4[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double a = (double)fabsf(w[j]);
        const double d6 = __builtin_fma(-cs6, (double)fabsf(q6[j]), a);
        const double d4 = __builtin_fma(-cs4, (double)fabsf(q4[j]), a);
        sq6[j] = d6 * d6;
        sq4[j] = d4 * d4;
      }
      double s6 = 0.0, s4 = 0.0;
      if (!odd) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          s6 = s6 + sq6[j];
          s4 = s4 + sq4[j];
        }
      }
      s6 = __shfl_xor(s6, 1);
      s4 = __shfl_xor(s4, 1);
      if (odd) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          s6 = s6 + sq6[j];
          s4 = s4 + sq4[j];
        }
      }
      const int pick4 = (odd && s4 < s6) ? 1 : 0;
      const int use4 = __shfl(pick4, (int)(threadIdx.x | 1) & 63);  // the odd lane decides
      if (use4) {
        word = word4;
        sc = k4;
      }
    }
    __builtin_nontemporal_store(word, &codes[h]);
    const uint32_t s1 = __shfl_down(sc, 2), s2 = __shfl_down(sc, 4), s3 = __shfl_down(sc, 6);
    if (pack && (h | 7) < n_half) {
      if ((h & 7) == 0) reinterpret_cast<uint32_t*>(scales)[h >> 3] = sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
    } else if ((h & 1) == 0) {
      scales[h >> 1] = (uint8_t)sc;
    }
  }
}

hipError_t launch_quantize_4o6(const void* x, bool bf16, int64_t n_elems, const float* sg, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
  int64_t n_half = n_elems / 8;
  if (n_half == 0) return hipSuccess;
  int64_t wg = (n_half + 255) / 256;
  if (wg > 8192) wg = 8192;
  if (bf16)
    hipLaunchKernelGGL(quantize_4o6_kernel<true>, dim3((unsigned)wg), dim3(256), 0, stream, x, n_half, sg,
                       reinterpret_cast<uint32_t*>(codes), scales);
  else
    hipLaunchKernelGGL(quantize_4o6_kernel<false>, dim3((unsigned)wg), dim3(256), 0, stream, x, n_half, sg,
                       reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_quantize_absmax(const void* x, bool bf16, int64_t n_elems, const float* sg, uint8_t* codes,
                                  uint8_t* scales, hipStream_t stream) {
  int64_t n_half = n_elems / 8;
  if (n_half == 0) return hipSuccess;
  int64_t wg = (n_half + 255) / 256;
  if (wg > kQuantizeMaxGrid) wg = kQuantizeMaxGrid;
  if (bf16)
    hipLaunchKernelGGL(quantize_absmax_kernel<true>, dim3((unsigned)wg), dim3(256), 0, stream, x, n_half, sg,
                       reinterpret_cast<uint32_t*>(codes), scales);
  else
    hipLaunchKernelGGL(quantize_absmax_kernel<false>, dim3((unsigned)wg), dim3(256), 0, stream, x, n_half, sg,
                       reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

}  // namespace nvfp4
