// W4A16 decode product y = x W^^T for NVFP4 weights and bf16 activations,
// M <= 16 rows ("Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de
// laptop", section 2: W4A16 stores 4-bit weights and unpacks them to 16 bits
// for the multiply; decoding reads every weight once per token).
//
// Design (gfx950): the kernel streams the packed weights from HBM exactly
// once with 16-byte loads.  A workgroup of 4 waves owns 64 weight rows and a
// K range; its slice of x (M rows) sits in LDS.  Each wave computes a
// 16 (m) x 16 (n) tile with v_mfma_f32_16x16x32_bf16: lane (n, h) unpacks 32
// codes of row n into bf16 values q * s_b (exact: <= 6 significant bits,
// magnitudes in [2^-10, 2688]) and lane (m, h) feeds the matching x values;
// the k order inside a 32-wide MFMA step is the same for both operands, so
// any assignment of k to lanes is valid.  fp32 accumulation; the fp32
// epilogue multiplies by s_g and rounds to bf16 (RNE).  When the K range is
// split across workgroups, fp32 partial sums go to the workspace and a small
// reduce kernel adds them in split order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

namespace {
constexpr int kRowsPerWG = 64;  // 4 waves x 16 rows
constexpr int kRound = 128;     // k per round: 4 lane groups x 32
constexpr int kLdsPad = 8;      // bf16 elements of padding per LDS row
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

// grid: (ceil(N / 64), splits); block 256; dynamic LDS M * (kc + 8) * 2 bytes.
// mode 0: y = bf16(acc * s_g); 1: y = fp32(acc * s_g); 2: partial[split] = acc.
__global__ __launch_bounds__(256) void gemv_w4a16_kernel(const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ sg_ptr, int M, int N, int K,
                                                         int kc, int mode, void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  const int kbeg = blockIdx.y * kc;
  const int klen = min(kc, K - kbeg);
  const int ldw = kc + kLdsPad;

  // Stage x[0:M, kbeg:kbeg+klen] in LDS (16-byte chunks).
  {
    const int chunks_per_row = klen / 8;
    const int total = M * chunks_per_row;
    for (int t = threadIdx.x; t < total; t += blockDim.x) {
      int m = t / chunks_per_row, c = t - m * chunks_per_row;
      u32x4 v = *reinterpret_cast<const u32x4*>(x + (int64_t)m * K + kbeg + 8 * c);
      *reinterpret_cast<u32x4*>(xs + m * ldw + 8 * c) = v;
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nl = lane & 15;  // weight row within the tile (B column) / x row (A row)
  const int h = lane >> 4;   // lane group: k sub-range 32h .. 32h+31 of each round
  const int row0 = blockIdx.x * kRowsPerWG + wave * 16;
  const int row = min(row0 + nl, N - 1);
  const uint8_t* crow = codes + (int64_t)row * (K / 2);
  const uint8_t* srow = scales + (int64_t)row * (K / 16);
  const bool a_live = nl < M;
  const uint16_t* xrow = xs + nl * ldw;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int nround = (klen + kRound - 1) / kRound;
  constexpr int U = 4;  // rounds per load group
  for (int r0 = 0; r0 < nround; r0 += U) {
    u32x4 cw[U];
    uint32_t sw[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int kk = (r0 + u) * kRound + 32 * h;  // offset inside the K range
      live[u] = (r0 + u < nround) && (kk < klen);
      int kg = kbeg + (live[u] ? kk : 0);
      cw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + kg / 2));
      sw[u] = *reinterpret_cast<const uint16_t*>(srow + kg / 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (r0 + u >= nround) break;
      int kk = (r0 + u) * kRound + 32 * h;
      float sb0 = e4m3_to_f32(sw[u] & 0xFFu), sb1 = e4m3_to_f32(sw[u] >> 8);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 b = live[u] ? unpack8_bf16(cw[u][s], s < 2 ? sb0 : sb1) : bf16x8{};
        bf16x8 a = {};
        if (live[u] && a_live) a = *reinterpret_cast<const bf16x8*>(xrow + kk + 8 * s);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
      }
    }
  }

  // acc[i] holds C[m = 4h + i][n = nl].
  const float sg = *sg_ptr;
  const int n = row0 + nl;
  if (n < N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int m = 4 * h + i;
      if (m >= M) continue;
      if (mode == 0) {
        reinterpret_cast<uint16_t*>(out)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(acc[i] * sg);
      } else if (mode == 1) {
        reinterpret_cast<float*>(out)[(int64_t)m * N + n] = acc[i] * sg;
      } else {
        reinterpret_cast<float*>(out)[((int64_t)blockIdx.y * M + m) * N + n] = acc[i];
      }
    }
  }
}

// y[m, n] = round(s_g * sum_s partial[s, m, n]), sum in split order.
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ partial, int splits, int64_t mn,
                                                          const float* __restrict__ sg_ptr, int bf16_out,
                                                          void* __restrict__ out) {
  const float sg = *sg_ptr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int p = 0; p < splits; ++p) s += partial[p * mn + i];
    if (bf16_out)
      reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(s * sg);
    else
      reinterpret_cast<float*>(out)[i] = s * sg;
  }
}

// K split and chunk: enough workgroups to cover the CUs, LDS slice <= 64 KB.
void gemv_plan(int64_t M, int64_t N, int64_t K, int* splits, int* kc) {
  int64_t groups = (N + kRowsPerWG - 1) / kRowsPerWG;
  int64_t max_kc = (65536 / (2 * (M > 0 ? M : 1)) - kLdsPad) / kRound * kRound;
  if (max_kc < kRound) max_kc = kRound;
  int64_t s = 1;
  while (groups * s < 256 && s < 8) s *= 2;
  int64_t c = (K + s - 1) / s;
  c = (c + kRound - 1) / kRound * kRound;
  if (c > max_kc) c = max_kc;
  s = (K + c - 1) / c;
  *splits = (int)s;
  *kc = (int)c;
}

size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  int s, c;
  gemv_plan(M, N, K, &s, &c);
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

hipError_t launch_gemv_w4a16(const uint16_t* x, const uint8_t* codes, const uint8_t* scales, const float* sg,
                             int64_t M, int64_t N, int64_t K, void* y, bool bf16_out, float* partial,
                             hipStream_t stream) {
  int splits, kc;
  gemv_plan(M, N, K, &splits, &kc);
  dim3 grid((unsigned)((N + kRowsPerWG - 1) / kRowsPerWG), (unsigned)splits);
  size_t lds = (size_t)M * (kc + kLdsPad) * 2;
  int mode = splits > 1 ? 2 : (bf16_out ? 0 : 1);
  void* dst = splits > 1 ? (void*)partial : y;
  hipLaunchKernelGGL(gemv_w4a16_kernel, grid, dim3(256), lds, stream, x, codes, scales, sg, (int)M, (int)N, (int)K,
                     kc, mode, dst);
  if (splits > 1) {
    int64_t mn = M * N;
    int64_t wg = (mn + 255) / 256;
    if (wg > 4096) wg = 4096;
    hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)wg), dim3(256), 0, stream, partial, splits, mn, sg,
                       bf16_out ? 1 : 0, y);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
