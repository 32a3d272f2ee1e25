// NVFP4 dequantization W^ = q * s_b * s_g ("Tu pipeline NVFP4: meter 62 GB de
// modelo en 24 GB de laptop", section 2, hierarchical reconstruction).
// q * s_b is exact in fp32; the product with s_g rounds once; bf16 output is
// the nearest-even rounding of that fp32 value.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

// One lane per 8 elements (one dword of codes).
template <bool kBF16Out>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ sg_ptr, int64_t n_oct,
                                                      void* __restrict__ out) {
  const float sg = *sg_ptr;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; h < n_oct; h += stride) {
    uint32_t c = codes[h];
    float sb = e4m3_to_f32(scales[h >> 1]);
    float v[8];
    fp4x8_to_f32(c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (v[j] * sb) * sg;
    if constexpr (kBF16Out) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x2 p = {(__bf16)v[2 * j], (__bf16)v[2 * j + 1]};
        o[j] = __builtin_bit_cast(uint32_t, p);
      }
      reinterpret_cast<u32x4*>(out)[h] = o;
    } else {
      u32x4* o = reinterpret_cast<u32x4*>(out) + 2 * h;
      o[0] = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
      o[1] = u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
    }
  }
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* sg, int64_t n_elems,
                          void* out, bool bf16_out, hipStream_t stream) {
  int64_t n_oct = n_elems / 8;
  if (n_oct == 0) return hipSuccess;
  int64_t wg = (n_oct + 255) / 256;
  if (wg > 8192) wg = 8192;
  const uint32_t* c = reinterpret_cast<const uint32_t*>(codes);
  if (bf16_out)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)wg), dim3(256), 0, stream, c, scales, sg, n_oct, out);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)wg), dim3(256), 0, stream, c, scales, sg, n_oct, out);
  return hipGetLastError();
}

}  // namespace nvfp4
