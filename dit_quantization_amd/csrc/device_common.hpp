// Device-side helpers shared by the gfx950 NVFP4 kernels.
//
// Format facts used here ("Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB
// de laptop", section 2): E2M1 codes (sign bit 3, magnitudes 0, .5, 1, 1.5, 2,
// 3, 4, 6), 16-element blocks along the reduction dimension, one E4M3 scale
// per block, one fp32 scale per tensor, W^ = q * s_b * s_g.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Largest E4M3 ("fn") value and its code; 6 * 448 sets the per-tensor scale.
constexpr double kE4M3Max = 448.0;
constexpr uint32_t kE4M3MaxCode = 126u;
constexpr double kGlobalDiv = 2688.0;

// Fast-path ambiguity window for E2M1 rounding of an approximate fp32
// quotient: +-64 ulps around every value with <= 2 fraction bits (this
// includes every E2M1 midpoint 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5).
constexpr uint32_t kNearUlps = 64u;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 byte (non-negative, 0x00..0x7E) -> exact fp32 value.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
  float sub = (float)m * 0.001953125f;  // m * 2^-9
  return e ? normal : sub;
}

// Nearest non-negative E4M3 code to a >= 0 (a the correctly rounded fp64
// quotient amax / (6 s_g)), ties to the even code, saturating at 448.
// fp64 is wide enough that rounding the quotient to fp64 first never moves
// it across an E4M3 midpoint.
__device__ __forceinline__ uint32_t e4m3_code_rne(double a) {
  if (a >= kE4M3Max) return kE4M3MaxCode;
  if (a < 0.015625) return (uint32_t)__builtin_rint(a * 512.0);  // subnormal step 2^-9
  int E;
  double f = __builtin_frexp(a, &E);                               // a = f 2^E, f in [0.5, 1)
  double mant = __builtin_rint((f * 2.0 - 1.0) * 8.0);             // 0..8 (8 carries)
  return (uint32_t)((E + 6) * 8 + (int)mant);
}

// Per-tensor scale from the tensor amax: fp32(amax / 2688), 1 for zero.
__device__ __forceinline__ float global_scale_from_amax(float amax) {
  if (amax == 0.0f) return 1.0f;
  return (float)((double)amax / kGlobalDiv);
}

// Exact E2M1 code of w for the (exact, fp64) divisor D = s_b * s_g:
// compare |w| with the midpoints m_j * D (products exact in fp64).  Ties go
// to the even code; zero magnitude is always code 0.
__device__ __forceinline__ uint32_t e2m1_code_exact(float w, double D) {
  double aw = __builtin_fabs((double)w);
  uint32_t idx = (aw > 0.25 * D) + (aw >= 0.75 * D) + (aw > 1.25 * D) + (aw >= 1.75 * D) +
                 (aw > 2.5 * D) + (aw >= 3.5 * D) + (aw > 5.0 * D);
  return idx == 0 ? 0u : (idx | (w < 0.0f ? 8u : 0u));
}

// True when the approximate quotient x may lie within rounding error of an
// E2M1 rounding boundary (only magnitudes >= 0.125 can).
__device__ __forceinline__ bool e2m1_near_boundary(float x) {
  uint32_t b = __float_as_uint(x) & 0x7FFFFFFFu;
  return (b >= 0x3E000000u) && (((b + kNearUlps) & 0x1FFFFFu) < 2u * kNearUlps);
}

// Two fp32 values -> two E2M1 codes (RNE, saturating) placed in byte `sel`
// of `old` (low nibble = first value).  Scale 1.0: no extra scaling.
#define NVFP4_CVT_PK_FP4(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// Decode the 8 E2M1 codes of a dword (element j in bits 4j..4j+3) to exact
// fp32 / fp16 values (the converter's byte selector must be a constant).
__device__ __forceinline__ void fp4x8_to_f32(uint32_t c, float v[8]) {
  f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
  f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
  f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
  f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
  v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
  v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
}

__device__ __forceinline__ void fp4x8_to_f16x2(uint32_t c, f16x2 v[4]) {
  v[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0);
  v[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1);
  v[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2);
  v[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3);
}

// Clear the sign bit of every nibble whose magnitude is zero (no -0 codes).
__device__ __forceinline__ uint32_t canonical_zero_nibbles(uint32_t w) {
  uint32_t mag = w & 0x77777777u;
  uint32_t nz = (mag + 0x77777777u) & 0x88888888u;
  return w & (nz | 0x77777777u);
}

// Encode 8 elements of one block with block scale value sb (an exact E4M3
// value) and tensor scale sg into one dword (8 nibbles, element 0 in bits
// 0..3).  Fast path: x = w * (1/(sb sg)) in fp32 and the hardware RNE
// converter; elements whose approximate quotient lies near a rounding
// boundary, and blocks whose reciprocal is out of the fp32 fast range, take
// the exact fp64 comparison.  Codes of zero magnitude are canonical +0.
__device__ __forceinline__ uint32_t encode8(const float* w, float sb, float sg, float inv_sg) {
  if (sb == 0.0f) return 0u;
  double D = (double)sb * (double)sg;  // exact
  float inv = __builtin_amdgcn_rcpf(sb) * inv_sg;
  bool fast = inv < 0x1p100f && inv > 0x1p-100f;
  float x[8];
  bool near_any = !fast;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = w[j] * inv;
    near_any |= e2m1_near_boundary(x[j]);
  }
  uint32_t word = 0;
  word = NVFP4_CVT_PK_FP4(word, x[0], x[1], 0);
  word = NVFP4_CVT_PK_FP4(word, x[2], x[3], 1);
  word = NVFP4_CVT_PK_FP4(word, x[4], x[5], 2);
  word = NVFP4_CVT_PK_FP4(word, x[6], x[7], 3);
  word = canonical_zero_nibbles(word);
  if (near_any) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!fast || e2m1_near_boundary(x[j])) {
        uint32_t c = e2m1_code_exact(w[j], D);
        word = (word & ~(0xFu << (4 * j))) | (c << (4 * j));
      }
    }
  }
  return word;
}

// Raw buffer access (gfx9 buffer resource, stride 0): a load whose byte
// offset is at or past `bytes` returns zero without touching memory, which
// replaces clamped addresses and select masks for tails and idle lanes.
constexpr int kBufOOB = 0x40000000;  // an offset past every buffer the kernels address this way
constexpr int kBufNT = 2;            // aux bit: non-temporal (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buf(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// SVDQuant smoothing of 8 bf16 values (packed in v) by the per-channel fp32
// multipliers m[0..7]: bf16(fp32(x * m)), both roundings to nearest even
// (the fp32 product of a bf16 and an fp32 is correctly rounded).
__device__ __forceinline__ u32x4 smooth8(u32x4 v, f32x4 m0, f32x4 m1) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = bf16_bits_to_f32(v[j] & 0xFFFFu) * (j < 2 ? m0[2 * j] : m1[2 * j - 4]);
    const float b = bf16_bits_to_f32(v[j] >> 16) * (j < 2 ? m0[2 * j + 1] : m1[2 * j - 3]);
    o[j] = f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
  }
  return o;
}

// s_waitcnt immediate for vmcnt(n) with lgkmcnt(0) (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt left at its maximum 7).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// 16 (2) bytes per lane from a buffer straight into LDS: lane i of the wave
// writes 16 bytes at lds_base + 16 i (the 2 bytes zero-extended to the dword
// at lds_base + 4 i); offsets past the buffer write zeros.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t buf, u32x4* lds_base, uint32_t voff,
                                                uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(buf, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buffer_to_lds2(__amdgpu_buffer_rsrc_t buf, uint32_t* lds_base, uint32_t voff,
                                               uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(buf, (__attribute__((address_space(3))) void*)lds_base, 2, voff, soff, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace nvfp4
