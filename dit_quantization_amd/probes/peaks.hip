// Reference-rate probes for the benchmark: what this GPU reaches on plain
// work, measured next to the datasheet peaks.  Not part of the NVFP4 path.
//  * probe_mfma_f16: back-to-back v_mfma_f32_32x32x16_f16 (the W4A4
//    product's instruction) on register operands, no memory traffic: the
//    matrix cores' achievable dense fp16 rate at the running clock.
//  * probe_read: a streaming 16-byte-load read of a buffer (each byte once,
//    several loads in flight per lane): the achievable HBM read rate for a
//    given size (a 33 MB decode weight, or a large buffer).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_f16_loop_kernel(float* __restrict__ out, int iters) {
  f16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(float)((threadIdx.x + j) & 7);
    b[j] = (_Float16)(float)((threadIdx.x * 3 + j) & 7);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][c];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the loop live
}

// Each workgroup streams one contiguous segment of the buffer (the layout
// the decode kernels read weights in): lane l takes 16-byte vectors
// l, l + 256, ... of the segment, four loads in flight per iteration; one
// xor per workgroup is written so the loads stay.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n_vec,
                                                   uint32_t* __restrict__ out) {
  const int64_t per = (n_vec + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n_vec ? beg + per : n_vec;
  int64_t i = beg + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + 256);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 512);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 768);
    x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w ^ v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < end; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[4];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

extern "C" {

// FLOPs of one probe_mfma_f16 launch: blocks * 4 waves * iters * kChains *
// 32 * 32 * 16 * 2.  out: blocks * 256 floats.  Returns a hipError_t code.
int probe_mfma_f16(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_f16_loop_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), out, iters);
  return (int)hipGetLastError();
}

double probe_mfma_f16_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
}

// Reads `bytes` (a multiple of 16, 16-byte aligned) from src; out: `blocks`
// uint32.  Returns a hipError_t code.
int probe_read(const void* src, int64_t bytes, uint32_t* out, int blocks, void* stream) {
  if (!src || !out || bytes <= 0 || (bytes & 15) || blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const u32x4*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
