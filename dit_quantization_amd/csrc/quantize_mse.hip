// NVFP4 quantizer with MSE-searched block scales for gfx950.
//
// "Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de laptop", section 2,
// box "Derivacion del objetivo de optimizacion MSE vs Absmax": the block
// scale minimises sum_k (W_k - s_b s_g Q(W_k / (s_b s_g)))^2; the algorithm
// table: MSE tries several scales and keeps the one with the least block
// reconstruction error (accepting some clipping of the largest value in
// exchange for finer steps on the other fifteen).
//
// Candidate set (fixed by this library): the absmax scale plus every
// positive E4M3 value c with a/2 <= c <= min(2a, 448), a = amax / (6 s_g),
// tested exactly as m <= 12 s_g c and 3 s_g c <= m in fp64.  Error:
// d_k = |W_k| - c s_g |q_k| (exact or rounded once), E = ((d_0^2 + d_1^2) +
// ...) + d_15^2 in fp64, one rounding per operation; candidates in ascending
// order, replaced only on a strictly smaller error.
//
// Design: the search is ALU work, so one lane owns one 16-element block and
// walks its ~16 candidates with no cross-lane traffic.  Each lane iterates
// over its own candidate list (the wave runs as many iterations as its
// longest list, not the union of the lanes' code ranges).  Element codes per
// candidate come from the hardware E2M1 converter applied to the fp32
// quotient x = |W| (1 / c) (1 / s_g), whose relative error is below 3 ulps.
// Every E2M1 rounding midpoint has at most 3 significant bits, so when no
// x of the block lies within 8 ulps of a number whose low 21 mantissa bits
// are zero, x and the exact quotient round alike and the fast codes stand;
// otherwise (rare) the block's codes for that candidate come from exact fp64
// comparisons.  The error terms are computed in fp64 exactly as specified.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {
// ((bits(x) + 8) << 11) < (16 << 11)  <=>  the low 21 mantissa bits of x
// are within -8..+7 of zero (mod 2^21).  Zero inputs get bit 20 added so
// that they never test positive.
constexpr uint32_t kNearOff = 8u << 11;
constexpr uint32_t kZeroOff = (0x00100000u + 8u) << 11;
constexpr uint32_t kNearLim = 16u << 11;
}  // namespace

template <bool kBF16>
__device__ __forceinline__ void load16(const void* __restrict__ x, int64_t b, float w[16]) {
  if constexpr (kBF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(x) + 2 * b;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 v = __builtin_nontemporal_load(p + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[8 * i + 2 * j] = bf16_bits_to_f32(v[j] & 0xFFFFu);
        w[8 * i + 2 * j + 1] = bf16_bits_to_f32(v[j] >> 16);
      }
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(x) + 4 * b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 v = __builtin_nontemporal_load(p + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) w[4 * i + j] = __uint_as_float(v[j]);
    }
  }
}

// kFourOverSix: the candidates are only the scales that map the block
// maximum onto 6 (absmax) and onto 4 ("Tu pipeline NVFP4 ...", section 2,
// algorithm table: four-over-six), same error and tie rule.
template <bool kBF16, bool kFourOverSix>
__global__ __launch_bounds__(256) void quantize_mse_kernel(const void* __restrict__ x, int64_t nblocks,
                                                           const float* __restrict__ sg_ptr,
                                                           u32x2* __restrict__ codes, uint8_t* __restrict__ scales) {
  const float sg = *sg_ptr;
  const float inv_sg = 1.0f / sg;
  const double sg64 = (double)sg;
  const double six_sg = 6.0 * sg64;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
    float w[16], aw[16];
    load16<kBF16>(x, b, w);
    float mf = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      aw[k] = fabsf(w[k]);
      mf = fmaxf(mf, aw[k]);
    }
    const double m = (double)mf;
    const double a = m / six_sg;
    const int kabs = (int)e4m3_code_rne(a);
    int klo = 0, khi = 0, kfirst = kabs, ncand = 1, k4 = kabs;
    if (kFourOverSix) {
      k4 = (int)e4m3_code_rne(m / (4.0 * sg64));  // >= kabs
      ncand = k4 != kabs ? 2 : 1;
    } else {
      // Window [k_lo, k_hi] of codes c >= 1 with a/2 <= c <= 2a (exact tests).
      klo = (int)e4m3_code_rne(a * 0.5);
      if (klo < 1) klo = 1;
      if (12.0 * sg64 * (double)e4m3_to_f32(klo) < m) ++klo;
      if (klo > 1 && 12.0 * sg64 * (double)e4m3_to_f32(klo - 1) >= m) --klo;
      khi = (int)e4m3_code_rne(a * 2.0);
      if (khi >= 1 && 3.0 * sg64 * (double)e4m3_to_f32(khi) > m) --khi;
      if (khi < (int)kE4M3MaxCode && 3.0 * sg64 * (double)e4m3_to_f32(khi + 1) <= m) ++khi;
      kfirst = min(klo, kabs);
      ncand = max(khi, kabs) - kfirst + 1;
    }

    double aw64[16];
    uint32_t zoff[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      aw64[e] = (double)aw[e];
      zoff[e] = aw[e] == 0.0f ? kZeroOff : kNearOff;
    }

    double best_err = 0.0;
    int best = -1;
    for (int i = 0; i < ncand; ++i) {
      const int k = kFourOverSix ? (i == 0 ? kabs : k4) : kfirst + i;
      if (!kFourOverSix && (k < klo || k > khi) && k != kabs) continue;
      double err = 0.0;
      if (k == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) err = err + aw64[e] * aw64[e];
      } else {
        const float c = e4m3_to_f32((uint32_t)k);
        const double cs = (double)c * sg64;  // exact
        const float inv = __builtin_amdgcn_rcpf(c) * inv_sg;
        float q[16];
        uint32_t tmin = 0xFFFFFFFFu;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float xs[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xs[e] = aw[8 * h + e] * inv;
            tmin = min(tmin, (__float_as_uint(xs[e]) << 11) + zoff[8 * h + e]);
          }
          uint32_t word = 0;
          word = NVFP4_CVT_PK_FP4(word, xs[0], xs[1], 0);
          word = NVFP4_CVT_PK_FP4(word, xs[2], xs[3], 1);
          word = NVFP4_CVT_PK_FP4(word, xs[4], xs[5], 2);
          word = NVFP4_CVT_PK_FP4(word, xs[6], xs[7], 3);
          fp4x8_to_f32(word, q + 8 * h);
        }
        const bool fast = inv < 0x1p100f && inv > 0x1p-100f;
        if (!fast || tmin < kNearLim) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const f32x2 ex = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(e2m1_code_exact(aw[e], cs), 1.0f, 0);
            q[e] = ex.x;
          }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          // |W| - c s_g |q|: c s_g q is exact, so the fused form rounds once,
          // like the separate subtraction of the exact product.
          const double d = __builtin_fma(-cs, (double)q[e], aw64[e]);
          const double sq = d * d;
          err = err + sq;
        }
      }
      if (best < 0 || err < best_err) {
        best = k;
        best_err = err;
      }
    }
    const float sb = e4m3_to_f32((uint32_t)best);
    u32x2 out;
    out.x = encode8(w, sb, sg, inv_sg);
    out.y = encode8(w + 8, sb, sg, inv_sg);
    __builtin_nontemporal_store(out, &codes[b]);
    scales[b] = (uint8_t)best;
  }
}

hipError_t launch_quantize_search(const void* x, bool bf16, bool four_over_six, int64_t n_elems, const float* sg,
                                  uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  int64_t nb = n_elems / 16;
  if (nb == 0) return hipSuccess;
  int64_t wg = (nb + 255) / 256;
  if (wg > 16384) wg = 16384;
  u32x2* c = reinterpret_cast<u32x2*>(codes);
#define NVFP4_QSEARCH(B, F) \
  hipLaunchKernelGGL((quantize_mse_kernel<B, F>), dim3((unsigned)wg), dim3(256), 0, stream, x, nb, sg, c, scales)
  if (bf16) {
    if (four_over_six) NVFP4_QSEARCH(true, true);
    else NVFP4_QSEARCH(true, false);
  } else {
    if (four_over_six) NVFP4_QSEARCH(false, true);
    else NVFP4_QSEARCH(false, false);
  }
#undef NVFP4_QSEARCH
  return hipGetLastError();
}

}  // namespace nvfp4
