// W4A4 GEMM with online NVFP4 activation quantization for gfx950.
//
// "NVFP4 en difusion: la misma cuantizacion, un motor completamente
// distinto", section 2 ("NVFP4 sin vLLM: torch._scaled_mm a mano"): the
// activation is quantized to NVFP4 on every call, 16-element block by block
// with the absmax criterion, and out = (A s_a)(B s_b)^T is returned in 16-bit
// precision (a "4-bit island with BF16 shores").
//
// Design (gfx950):
//  * act_quant: absmax NVFP4 quantization of A (same encoder as the weight
//    quantizer), written out as the exact fp16 values q_a * s_a (<= 6
//    significant bits, magnitudes in [2^-10, 2688], so fp16 holds them
//    exactly and the bf16/fp16 matrix cores can consume them directly).
//  * gemm: 256x256 (or 128x128) output tiles per workgroup of 4 waves in a
//    2x2 arrangement, K step 64.  A^ tiles go global -> registers -> LDS
//    (XOR-swizzled 16-byte chunks, double buffered).  Packed weights go
//    global -> registers; each lane unpacks its 32 codes with the hardware
//    FP4 converter and one packed fp16 multiply by the block scale, giving
//    exact fp16 q_w * s_w operands.  v_mfma_f32_32x32x16_f16 accumulates in
//    fp32 (every product is exact); the epilogue multiplies by
//    fp32(s_gA * s_gW) and rounds to bf16.
//  * The k order inside each 64-wide K step is permuted identically for A
//    and W (lane group g of an MFMA feeds k = 32 g + 8 s + j at sub-step s),
//    which lets every lane read 16 contiguous bytes of packed weights.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- act quant

// One lane per half block of the bf16 activation; lanes 2b, 2b+1 share block b.
__global__ __launch_bounds__(256) void act_quant_f16_kernel(const u32x4* __restrict__ a, int64_t n_half,
                                                            const float* __restrict__ sg_ptr,
                                                            u32x4* __restrict__ a_hat) {
  const float sg = *sg_ptr;
  const float inv_sg = 1.0f / sg;
  const double six_sg = 6.0 * (double)sg;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; h < n_half; h += stride) {
    u32x4 v = __builtin_nontemporal_load(&a[h]);
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
    a_hat[h] = o;
  }
}

hipError_t launch_act_quant_f16(const uint16_t* a, int64_t n_elems, const float* sg, uint16_t* a_hat,
                                hipStream_t stream) {
  int64_t n_half = n_elems / 8;
  if (n_half == 0) return hipSuccess;
  int64_t wg = (n_half + 255) / 256;
  if (wg > 8192) wg = 8192;
  hipLaunchKernelGGL(act_quant_f16_kernel, dim3((unsigned)wg), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(a), n_half, sg, reinterpret_cast<u32x4*>(a_hat));
  return hipGetLastError();
}

// ---------------------------------------------------------------- GEMM

namespace {
constexpr int BK = 64;  // K step (4 blocks of 16)
}

// Unpack 8 codes (one dword) into 8 exact fp16 values q * s_b.
__device__ __forceinline__ f16x8 unpack8_f16(uint32_t c, f16x2 s2) {
  f16x2 q[4];
  fp4x8_to_f16x2(c, q);
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f16x2 p = q[j] * s2;
    r[2 * j] = p.x;
    r[2 * j + 1] = p.y;
  }
  return r;
}

// Two E4M3 scale bytes (bits 0..15) -> fp16 values with the hardware
// converter (exact: every E4M3 value, subnormals included, is a normal fp16
// number; the E4M3 decode is checked exhaustively by the dequant tests).
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t b) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
}

// BM x BN tile per workgroup of WM x WN waves; each wave (BM/WM) x (BN/WN)
// as TM x TN tiles of 32x32.  grid.x enumerates tiles (XCD-aware order).
// K loop: A tiles are double buffered in LDS and fetched two K steps ahead
// into one of two register sets; packed weights are fetched two K steps
// ahead into registers.  The loop is unrolled by two so every register set
// is addressed statically.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a4_kernel(const uint16_t* __restrict__ a_hat,
                                                                 const float* __restrict__ sga_ptr,
                                                                 const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ scales,
                                                                 const float* __restrict__ sgw_ptr, int M, int N,
                                                                 int K, void* __restrict__ y, int bf16_out) {
  constexpr int NT = WM * WN * 64;                       // threads
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;    // 32x32 tiles per wave
  constexpr int A_CHUNKS = BM * BK * 2 / 16;             // 16-byte chunks per A tile
  constexpr int APT = A_CHUNKS / NT;
  static_assert(A_CHUNKS % NT == 0, "A tile must split evenly over the threads");
  __shared__ __attribute__((aligned(16))) u32x4 lds_a[2][A_CHUNKS];

  // Tile coordinates.  Consecutive workgroup ids go to different XCDs
  // (round robin over 8); remap so each XCD receives a contiguous run of
  // tiles, which then share A rows / W rows in that XCD's L2.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) {  // a bijection on [0, ntiles) when 8 divides it
    const int per_xcd = ntiles >> 3;
    bid = (bid & 7) * per_xcd + (bid >> 3);
  }
  // Walk tiles in groups of 8 M-tiles so neighbouring workgroups reuse W.
  constexpr int GROUP = 8;
  const int group = bid / (GROUP * tiles_n);
  const int first_m = group * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % (GROUP * tiles_n)) % gsize;
  const int tn = (bid % (GROUP * tiles_n)) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, g = lane >> 5;  // MFMA row/col and k lane group

  // ---- A global -> LDS mapping: chunk tid + NT j -> row tid / 8 + j NT / 8,
  // 16-byte chunk tid % 8 of the row's 64 k; LDS slot XOR-swizzled by row.
  // NT / 8 is a multiple of 8, so every row of a thread has the same swizzle.
  const int a_r0 = tid >> 3, a_c = tid & 7;
  const int a_slot0 = a_r0 * 8 + (a_c ^ (a_r0 & 7));
  const u32x4* a_base = reinterpret_cast<const u32x4*>(a_hat) + a_c;

  // ---- W rows of this lane: TN sub-tiles, row n0 + wn*(BN/WN) + 32 t + l32
  const uint8_t* wc[TN];
  const uint8_t* wsc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    int n = min(n0 + wn * (BN / WN) + 32 * t + l32, N - 1);
    wc[t] = codes + (int64_t)n * (K / 2) + 16 * g;      // 32 codes = 16 bytes per K step
    wsc[t] = scales + (int64_t)n * (K / 16) + 2 * g;    // 2 scale bytes per K step
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.0f;

  const int KT = K / BK;
  u32x4 aset0[APT], aset1[APT];
  u32x4 wset0[TN], wset1[TN];
  uint32_t sset0[TN], sset1[TN];
  auto load_a = [&](u32x4 (&dst)[APT], int kt) {
    const int kk = min(kt, KT - 1) * (BK / 8);
#pragma unroll
    for (int j = 0; j < APT; ++j) {
      const int row = min(m0 + a_r0 + j * (NT / 8), M - 1);
      dst[j] = a_base[(int64_t)row * (K / 8) + kk];
    }
  };
  auto load_w = [&](u32x4 (&dw)[TN], uint32_t (&ds)[TN], int kt) {
    const int kk = min(kt, KT - 1);
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      dw[t] = *reinterpret_cast<const u32x4*>(wc[t] + kk * (BK / 2));
      ds[t] = *reinterpret_cast<const uint16_t*>(wsc[t] + kk * (BK / 16));
    }
  };
  auto store_a = [&](const u32x4 (&src)[APT], int buf) {
#pragma unroll
    for (int j = 0; j < APT; ++j) lds_a[buf][a_slot0 + j * NT] = src[j];
  };
  // one K step of 64 = 4 sub-steps of 16 from LDS buffer `buf`
  auto compute = [&](int buf, const u32x4 (&wr)[TN], const uint32_t (&sr)[TN]) {
    f16x2 sc0[TN], sc1[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      f16x2 s2 = e4m3x2_to_f16x2(sr[t]);
      sc0[t] = f16x2{s2.x, s2.x};
      sc1[t] = f16x2{s2.y, s2.y};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 afrag[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        int r = wm * (BM / WM) + 32 * i + l32;
        afrag[i] = __builtin_bit_cast(f16x8, lds_a[buf][r * 8 + ((4 * g + s) ^ (r & 7))]);
      }
      f16x8 bfrag[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) bfrag[t] = unpack8_f16(wr[t][s], s < 2 ? sc0[t] : sc1[t]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afrag[i], bfrag[t], acc[i][t], 0, 0, 0);
    }
  };

  // prologue: A(0) -> LDS buffer 0; A(1) in flight in aset0; W(0), W(1) in flight
  load_a(aset1, 0);
  load_w(wset0, sset0, 0);
  load_w(wset1, sset1, 1);
  store_a(aset1, 0);
  load_a(aset0, 1);
  for (int kt = 0; kt < KT; kt += 2) {
    {  // even step: LDS 0 holds A(kt); aset0 = A(kt+1); wset0 = W(kt)
      __syncthreads();
      u32x4 wcur[TN];
      uint32_t scur[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        wcur[t] = wset0[t];
        scur[t] = sset0[t];
      }
      load_a(aset1, kt + 2);
      load_w(wset0, sset0, kt + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(0, wcur, scur);
      __builtin_amdgcn_sched_barrier(0);
      store_a(aset0, 1);
    }
    if (kt + 1 < KT) {  // odd step: LDS 1 holds A(kt+1); aset1 = A(kt+2); wset1 = W(kt+1)
      __syncthreads();
      u32x4 wcur[TN];
      uint32_t scur[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        wcur[t] = wset1[t];
        scur[t] = sset1[t];
      }
      load_a(aset0, kt + 3);
      load_w(wset1, sset1, kt + 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(1, wcur, scur);
      __builtin_amdgcn_sched_barrier(0);
      store_a(aset1, 0);
    }
  }

  // ---- epilogue: acc[i][t][r] = C[row = 8 (r/4) + 4 g + r%4][col = l32]
  const float alpha = (*sga_ptr) * (*sgw_ptr);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int n = n0 + wn * (BN / WN) + 32 * t + l32;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * (BM / WM) + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m >= M) continue;
        float v = acc[i][t][r] * alpha;
        if (bf16_out)
          reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(v);
        else
          reinterpret_cast<float*>(y)[(int64_t)m * N + n] = v;
      }
    }
  }
}

hipError_t launch_gemm_w4a4(const uint16_t* a_hat, const float* sga, const uint8_t* codes, const uint8_t* scales,
                            const float* sgw, int64_t M, int64_t N, int64_t K, void* y, bool bf16_out,
                            hipStream_t stream) {
  // 256 x 256 tiles (8 waves, 128 x 64 per wave) whenever they cover at least
  // half of the 256 CUs; otherwise 128 x 128 tiles (4 waves) for more
  // parallelism on short activations (measured on the prefill and DiT shapes).
  const int b = bf16_out ? 1 : 0;
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= 128) {
    hipLaunchKernelGGL((gemm_w4a4_kernel<256, 256, 2, 4>), dim3((unsigned)t256), dim3(512), 0, stream, a_hat, sga,
                       codes, scales, sgw, (int)M, (int)N, (int)K, y, b);
  } else {
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    hipLaunchKernelGGL((gemm_w4a4_kernel<128, 128, 2, 2>), dim3((unsigned)t128), dim3(256), 0, stream, a_hat, sga,
                       codes, scales, sgw, (int)M, (int)N, (int)K, y, b);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
