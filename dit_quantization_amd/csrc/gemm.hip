// W4A4 GEMM with online NVFP4 activation quantization for gfx950.
//
// "NVFP4 en difusion: la misma cuantizacion, un motor completamente
// distinto", section 2 ("NVFP4 sin vLLM: torch._scaled_mm a mano"): the
// activation is quantized to NVFP4 on every call, 16-element block by block
// with the absmax criterion, and out = (A s_a)(B s_b)^T is returned in 16-bit
// precision, so each quantized layer takes and returns 16-bit tensors.
//
// Design (gfx950):
//  * the activation arrives quantized (act_quant.hip) as the exact fp16
//    values q_a * s_a (<= 6 significant bits, magnitudes in [2^-10, 2688]),
//    which the fp16 matrix cores consume directly.
//  * gemm: 256x256 output tiles per workgroup of 8 waves (128x64 each), or
//    128x128 tiles of 4 waves for short activations, K step 64.  A^ tiles,
//    packed weight codes and their scales go global -> LDS directly (buffer
//    loads with the LDS bit) into three stages fetched ahead; A^ chunks sit
//    XOR-swizzled so 16-byte fragment reads are conflict-free.  Each lane
//    unpacks its weight codes with the hardware FP4 converter and one packed
//    fp16 multiply by the block scale, giving exact fp16 q_w * s_w operands.
//    v_mfma_f32_32x32x16_f16 accumulates in fp32 (every product is exact);
//    the epilogue multiplies by fp32(s_gA * s_gW) and rounds to bf16.
//  * The k order inside each 64-wide K step is permuted identically for A
//    and W (lane group g of an MFMA feeds k = 32 g + 8 s + j at sub-step s),
//    which lets every lane read 16 contiguous bytes of packed weights.
#include "device_common.hpp"
#include "kernels.hpp"

namespace nvfp4 {

typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// s_waitcnt immediate: at most n vector memory operations outstanding, all
// LDS operations complete (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4 = 7 means no wait, lgkmcnt 11:8).

// BM x BN tile per workgroup of WM x WN waves; each wave (BM/WM) x (BN/WN)
// as TM x TN tiles of 32x32.  grid.x enumerates tiles (XCD-aware order).
// K loop, one step per 64 k.  Every operand goes global -> LDS directly
// (buffer loads with the LDS bit; rows past M or N read as zero) into three
// stages fetched two steps ahead, so no register holds data in flight:
//  * A^ (fp16): a lane's DMA target is fixed by its lane number, so each
//    lane fetches the 16-byte chunk that belongs in its LDS slot under an
//    XOR swizzle (conflict-free 16-byte fragment reads).
//  * packed weights: row r's 32 code bytes of the step sit in two 16-byte
//    slots, swapped for rows with bit 3 set (conflict-free reads); the 4
//    scale bytes of a row are contiguous.
// One barrier per step, after an explicit wait for this step's stage.  Each
// lane reads its weight chunk and scales once per step and unpacks 8 codes
// per MFMA sub-step (hardware FP4 -> fp16 converter, one packed multiply by
// the block scale); A fragments are read one sub-step ahead of their MFMAs.
// The loop is unrolled by 3 so the stages (separate LDS arrays) are
// addressed statically.
// LORA: the epilogue adds L lora_up^T (bf16 L [M, rank] from
// act_quant_lora_kernel, bf16 lora_up [N, rank]) with
// v_mfma_f32_32x32x16_bf16 after scaling the product by s_gA s_gW.
// SPLIT (short activations, never with LORA): workgroup b computes K range
// b % splits of tile b / splits and stores its unscaled fp32 sums in
// partial [splits, M, N]; gemm_splitk_reduce_kernel finishes the product.
// (A separate instantiation: folding the range offsets into the unsplit
// kernel cost it 3-5 % on the prefill and DiT shapes.)
//
// The body below computes tile `bid` (K range `split` of `splits`) of one
// product; gemm_w4a4_kernel maps workgroups of one product onto it,
// gemm_w4a4_group_kernel workgroups of several products (one launch).
template <int BM, int BN, int WM, int WN, bool LORA, bool SPLIT>
__device__ __forceinline__ void gemm_w4a4_tile(
    int bid, int split, const uint16_t* __restrict__ a_hat, const float* __restrict__ sga_ptr,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, const float* __restrict__ sgw_ptr, int M,
    int N, int K, void* __restrict__ y, int bf16_out, const uint16_t* __restrict__ lora_l,
    const uint16_t* __restrict__ lora_up, int rank, int splits, float* __restrict__ partial) {
  constexpr int NT = WM * WN * 64;                       // threads
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;    // 32x32 tiles per wave
  constexpr int A_CHUNKS = BM * BK * 2 / 16;             // 16-byte chunks per A stage
  constexpr int APT = A_CHUNKS / NT;                     // A DMA instructions per lane and step
  constexpr int W_CHUNKS = BN * 2;                       // 16-byte code chunks (and scale dwords) per W stage
  constexpr int WPT = W_CHUNKS / NT;                     // W DMA instructions per lane and step (each kind)
  static_assert(A_CHUNKS % NT == 0 && W_CHUNKS % NT == 0, "tile shape must match the thread count");
  constexpr int VM_STEP = APT + 2 * WPT;                 // vector memory instructions per lane and step
  struct Stage {
    u32x4 a[A_CHUNKS];
    u32x4 w[W_CHUNKS];
    uint32_t s[BN * 2];
  };
  // one array, so the epilogue can stage a 64 KB half tile across st0 and st1
  __shared__ __attribute__((aligned(16))) Stage stages[3];
  Stage& st0 = stages[0];
  Stage& st1 = stages[1];
  Stage& st2 = stages[2];

  // Tile coordinates (bid already remapped by the caller, see below).
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  // Walk tiles in groups of 4 M-tiles so the tiles an XCD runs together
  // share A row panels and W column panels in its L2 (measured on the
  // prefill shape: 401 MB fetched past L2 per launch with groups of 4,
  // 603 MB with 8, 1107 MB with 16; 4 was also the fastest).
  constexpr int GROUP = 4;
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
  const int kts = SPLIT ? (K / BK + splits - 1) / splits : K / BK;
  const int kt0 = SPLIT ? split * kts : 0;            // first K step of this workgroup's range
  const int KT = SPLIT ? min(kts, K / BK - kt0) : kts;  // K steps in the range (>= 1)

  // ---- DMA sources.  A: instruction j of wave w fills slots
  // [64 (w APT + j), +64); slot S holds row S / 8, 16-byte chunk
  // (S % 8) ^ ((row / 2) % 8) of the step's 64 k.  A 16-byte LDS read serves
  // 16 lanes (16 consecutive rows) at a time: rows 2j and 2j + 1 fall in the
  // two halves of the 64 banks and the 8 row pairs get 8 different chunks
  // (with the swizzle on row % 8, rows r and r + 8 collided: 2-way conflicts).
  // Panel bytes min(BM, M - m0) K 2 <= 256 * 2^22 * 2 = 2^31 (the largest K
  // the C ABI admits): computed unsigned, every offset below stays under it.
  const __amdgpu_buffer_rsrc_t abuf =
      make_buf(a_hat + (int64_t)m0 * K, (uint32_t)min(BM, M - m0) * (uint32_t)K * 2u);
  uint32_t a_off[APT];
#pragma unroll
  for (int j = 0; j < APT; ++j) {
    const int S = 64 * (wave * APT + j) + lane;
    const int r = S >> 3, c = (S & 7) ^ ((r >> 1) & 7);
    a_off[j] = ((uint32_t)r * (uint32_t)K + 8u * (uint32_t)c) * 2u;
  }
  // W codes: slot u (= tid + NT j) holds row u / 2, half (u % 2) ^ ((row >> 3) & 1).
  // Scales: dword slot u holds bytes 2 (u % 2) .. +2 of row u / 2.
  const int w_rows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t wbuf = make_buf(codes + (int64_t)n0 * (K / 2), (uint32_t)w_rows * (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t sbuf = make_buf(scales + (int64_t)n0 * (K / 16), (uint32_t)w_rows * (uint32_t)(K / 16));
  uint32_t w_off[WPT], s_off[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int u = tid + NT * j;
    w_off[j] = (uint32_t)(u >> 1) * (uint32_t)(K / 2) + 16u * (uint32_t)((u & 1) ^ ((u >> 4) & 1));
    s_off[j] = (uint32_t)(u >> 1) * (uint32_t)(K / 16) + 2u * (uint32_t)(u & 1);
  }

  auto dma = [&](Stage& stg, int kt) {
    const uint32_t k = (uint32_t)(kt0 + min(kt, KT - 1));
#pragma unroll
    for (int j = 0; j < APT; ++j) buffer_to_lds16(abuf, stg.a + 64 * (wave * APT + j), a_off[j], k * (BK * 2));
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      buffer_to_lds16(wbuf, stg.w + NT * j + 64 * wave, w_off[j], k * (BK / 2));
      buffer_to_lds2(sbuf, stg.s + NT * j + 64 * wave, s_off[j], k * (BK / 16));
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.0f;

  // A fragment of sub-step s for tile row i: row r = wm*(BM/WM) + 32 i + l32
  // (r % 8 == l32 % 8), chunk 4 g + s.  W chunk of tile column t: row
  // rw = wn*(BN/WN) + 32 t + l32, half g; scale bytes 2 g, 2 g + 1 of the row.
  int a_row8[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row8[i] = (wm * (BM / WM) + 32 * i + l32) * 8;
  const int a_sw = (l32 >> 1) & 7;
  int w_slot[TN], s_slot[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int rw = wn * (BN / WN) + 32 * t + l32;
    w_slot[t] = 2 * rw + (g ^ ((rw >> 3) & 1));
    s_slot[t] = 2 * rw + g;
  }

  // Operands of one K step (64 = 4 sub-steps of 16): each lane's weight
  // chunk and scales, A fragments and unpacked weights of the current and
  // next sub-step (software pipeline, double buffered).
  u32x4 wr[TN];
  f16x2 sc0[TN], sc1[TN];
  f16x8 af[2][TM], bf[2][TN];

  // Reads of a stage's weight chunk / scales and its sub-step 0 operands
  // into buffer 0.
  auto load_first = [&](const Stage& stg) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      wr[t] = stg.w[w_slot[t]];
      f16x2 s2 = e4m3x2_to_f16x2(stg.s[s_slot[t]]);
      sc0[t] = f16x2{s2.x, s2.x};
      sc1[t] = f16x2{s2.y, s2.y};
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = __builtin_bit_cast(f16x8, stg.a[a_row8[i] + ((4 * g) ^ a_sw)]);
#pragma unroll
    for (int t = 0; t < TN; ++t) bf[0][t] = unpack8_f16(wr[t][0], sc0[t]);
  };
  // MFMAs of sub-step s (operands in buffer s & 1); for s < 3 the operands of
  // s + 1 are read and unpacked meanwhile (sched_group_barrier pins the
  // interleave: each MFMA is followed by one LDS read and a few VALU ops).
  constexpr int kMFMA = 0x008, kVALU = 0x002, kDSR = 0x100;
  auto substep = [&](const Stage& stg, int s) {
    const int cb = s & 1, nb = cb ^ 1;
    if (s < 3) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[nb][i] = __builtin_bit_cast(f16x8, stg.a[a_row8[i] + ((4 * g + s + 1) ^ a_sw)]);
#pragma unroll
      for (int t = 0; t < TN; ++t) bf[nb][t] = unpack8_f16(wr[t][s + 1], s + 1 < 2 ? sc0[t] : sc1[t]);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cb][i], bf[cb][t], acc[i][t], 0, 0, 0);
    if (s < 3) {
#pragma unroll
      for (int q = 0; q < TM * TN; ++q) {
        __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
        if (q < TM) __builtin_amdgcn_sched_group_barrier(kDSR, 1, 0);
        if (q < 4) __builtin_amdgcn_sched_group_barrier(kVALU, 2 * TN, 0);
      }
    }
  };

  // Step kt (stage `cur` holds kt, `nxt` holds kt+1): sub-steps 0..2; then,
  // once every wave's reads of `cur` are done, the barrier that also
  // publishes `nxt`, the DMA of kt+3 into `cur`, and sub-step 3 overlapped
  // with the reads and first unpack of `nxt`.  Issued after the DMA of kt+1:
  // that of kt+2.
  auto step = [&](int kt, Stage& cur, const Stage& nxt) {
    substep(cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    substep(cur, 1);
    __builtin_amdgcn_sched_barrier(0);
    substep(cur, 2);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM_STEP));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    dma(cur, kt + 3);
    // With at least as many MFMAs in the last sub-step as DMA instructions
    // (256 x 256 tiles), the DMA is interleaved with them (one per MFMA:
    // prefill 367 -> 358 us on constant operands); otherwise it goes out as
    // one burst before them (faster for 128 x 128 tiles).
    constexpr bool kInterleaveDma = TM * TN >= VM_STEP;
    if (!kInterleaveDma) __builtin_amdgcn_sched_barrier(0);
    // sub-step 3 uses buffer 1; the next stage's first operands go to buffer 0
    substep(cur, 3);
    load_first(nxt);
    // reads first (one per MFMA), the unpack in the second half
    constexpr int kReads = TM + 2 * TN, kMF = TM * TN;
    constexpr int kVmem = 0x020;
#pragma unroll
    for (int q = 0; q < kMF; ++q) {
      if (kInterleaveDma && q < VM_STEP) __builtin_amdgcn_sched_group_barrier(kVmem, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kMFMA, 1, 0);
      if (q < kReads) __builtin_amdgcn_sched_group_barrier(kDSR, 1, 0);
      if (q >= kMF / 2) __builtin_amdgcn_sched_group_barrier(kVALU, (8 * TN + 6 + kMF / 2 - 1) / (kMF / 2), 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  dma(st0, 0);
  dma(st1, 1);
  dma(st2, 2);
  // stage 0 complete (two DMA groups issued after it), then published
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * VM_STEP));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_first(st0);
  __builtin_amdgcn_sched_barrier(0);
  int kt = 0;
  for (; kt + 3 <= KT; kt += 3) {
    step(kt + 0, st0, st1);
    step(kt + 1, st1, st2);
    step(kt + 2, st2, st0);
  }
  if (kt + 0 < KT) step(kt + 0, st0, st1);
  if (kt + 1 < KT) step(kt + 1, st1, st2);
  // Drain the DMA still in flight into LDS before the workgroup exits.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  // ---- epilogue: acc[i][t][r] = C[row = 8 (r/4) + 4 g + r%4][col = l32]
  const float alpha = (*sga_ptr) * (*sgw_ptr);
  if constexpr (LORA) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][t][r] *= alpha;
    // Rows past M and N read as zero; lane (row, g) feeds k = 16 kk + 8 g + j.
    const __amdgpu_buffer_rsrc_t lbuf = make_buf(lora_l + (int64_t)m0 * rank, (uint32_t)(min(BM, M - m0) * rank * 2));
    const __amdgpu_buffer_rsrc_t ubuf = make_buf(lora_up + (int64_t)n0 * rank, (uint32_t)(min(BN, N - n0) * rank * 2));
    for (int kk = 0; kk < rank; kk += 16) {  // uniform
      bf16x8 lf[TM], uf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        lf[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               lbuf, ((wm * (BM / WM) + 32 * i + l32) * rank + kk + 8 * g) * 2, 0, 0));
#pragma unroll
      for (int t = 0; t < TN; ++t)
        uf[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               ubuf, ((wn * (BN / WN) + 32 * t + l32) * rank + kk + 8 * g) * 2, 0, 0));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lf[i], uf[t], acc[i][t], 0, 0, 0);
    }
  }
  // bf16 output of a 256 x 256 tile with 16-byte aligned rows: each 128-row
  // half (the 4 waves with wm = h) goes through LDS (the free stages) and out
  // as 16-byte stores, 16 per lane instead of 128 two-byte ones (prefill
  // 385-390 -> 384 us, DiT block 919-931 -> 912-914 us; same bytes).  The
  // stores are non-temporal: y is not read again here, and keeping it out of
  // L2 leaves room for the A and W panels the other tiles share (prefill
  // 383 -> 380-382 us, DiT block 915 -> 890-893 us).
  if constexpr (!SPLIT && BM == 256 && BN == 256 && WM == 2) {
    if (bf16_out && (N & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
      static_assert(sizeof(Stage) * 2 >= 128 * 256 * 2, "a half tile fits in two stages");
      uint16_t* const half_tile = reinterpret_cast<uint16_t*>(&stages[0]);  // [128][256] bf16
      __builtin_amdgcn_s_barrier();  // every wave's stage reads are done (waited above)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (wm == h) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
                const int col = wn * (BN / WN) + 32 * t + l32;
                const float v = LORA ? acc[i][t][r] : acc[i][t][r] * alpha;
                half_tile[row * 256 + col] = (uint16_t)f32_to_bf16_bits(v);
              }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = tid / 32 + 16 * j, chunk = tid % 32;
          const int m = m0 + 128 * h + row, n = n0 + 8 * chunk;
          const u32x4 v = *reinterpret_cast<const u32x4*>(&half_tile[row * 256 + 8 * chunk]);
          if (m < M && n < N) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(y) + (int64_t)m * N + n));
        }
        __syncthreads();
      }
      return;
    }
  }
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
        if (SPLIT) {
          partial[((int64_t)split * M + m) * N + n] = acc[i][t][r];
          continue;
        }
        float v = LORA ? acc[i][t][r] : acc[i][t][r] * alpha;
        if (bf16_out)
          reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_bits(v);
        else
          reinterpret_cast<float*>(y)[(int64_t)m * N + n] = v;
      }
    }
  }
}

// Consecutive workgroup ids go to different XCDs (round robin over 8);
// remap so each XCD receives a contiguous run of tiles, which then share A
// rows / W rows in that XCD's L2 (a bijection on [0, ntiles) when 8
// divides ntiles).
__device__ __forceinline__ int xcd_contiguous(int bid, int ntiles) {
  if ((ntiles & 7) != 0) return bid;
  return (bid & 7) * (ntiles >> 3) + (bid >> 3);
}

template <int BM, int BN, int WM, int WN, bool LORA, bool SPLIT>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu((BM / WM) * (BN / WN) >= 128 * 128 ? 1 : 2))) void gemm_w4a4_kernel(
    const uint16_t* __restrict__ a_hat, const float* __restrict__ sga_ptr, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ sgw_ptr, int M, int N, int K, void* __restrict__ y,
    int bf16_out, const uint16_t* __restrict__ lora_l, const uint16_t* __restrict__ lora_up, int rank, int splits,
    float* __restrict__ partial) {
  const int ntiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int split = SPLIT ? (int)(blockIdx.x % splits) : 0;
  const int bid = SPLIT ? (int)(blockIdx.x / splits) : xcd_contiguous((int)blockIdx.x, ntiles);
  gemm_w4a4_tile<BM, BN, WM, WN, LORA, SPLIT>(bid, split, a_hat, sga_ptr, codes, scales, sgw_ptr, M, N, K, y,
                                              bf16_out, lora_l, lora_up, rank, splits, partial);
}

// Several independent products in one launch, each on 256 x 256 tiles
// ("NVFP4 en difusion ...", section 1: a double-stream DiT block runs the
// image and the text tokens through separate weights, so each layer is one
// product per stream).  The products' tiles are numbered end to end and
// remapped to XCDs as one range; a workgroup finds its product by the
// table's prefix of tile counts.  Filling one grid with every product of a
// phase keeps all CUs busy where a single product's last round would not.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a4_group_kernel(
    const GemmGroup g, int bf16_out) {
  const int total = g.tile_begin[g.n];
  const int bid = xcd_contiguous((int)blockIdx.x, total);
  int p = 0;
#pragma unroll
  for (int t = 1; t < kMaxGemmGroup; ++t) p += (t < g.n && bid >= g.tile_begin[t]) ? 1 : 0;
  gemm_w4a4_tile<BM, BN, WM, WN, false, false>(bid - g.tile_begin[p], 0, g.a_hat[p], g.sga[p], g.codes[p],
                                               g.scales[p], g.sgw[p], g.M[p], g.N[p], g.K[p], g.y[p], bf16_out,
                                               nullptr, nullptr, 0, 1, nullptr);
}

// y = round(fp32(s_gA s_gW) * (((p_0 + p_1) + ...) + p_{S-1})) per element.
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const float* __restrict__ partial, int splits,
                                                                 int64_t n, const float* __restrict__ sga_ptr,
                                                                 const float* __restrict__ sgw_ptr,
                                                                 void* __restrict__ y, int bf16_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = partial[i];
  for (int t = 1; t < splits; ++t) s += partial[t * n + i];
  const float v = s * ((*sga_ptr) * (*sgw_ptr));
  if (bf16_out)
    reinterpret_cast<uint16_t*>(y)[i] = (uint16_t)f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(y)[i] = v;
}

namespace {
int64_t tiles128(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 127) / 128); }
int64_t tiles256(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 255) / 256); }
}  // namespace

int gemm_max_splits(int64_t M, int64_t N) {
  // Short activations with fewer 128 x 128 tiles than CUs: enough K ranges
  // for about 384 workgroups, at most 8.
  if (M == 0 || N == 0 || tiles256(M, N) >= 128) return 1;
  const int64_t t = tiles128(M, N);
  if (t >= 256) return 1;
  const int64_t s = (384 + t - 1) / t;
  return (int)(s > 8 ? 8 : s);
}

int gemm_splits(int64_t M, int64_t N, int64_t K) {
  int s = gemm_max_splits(M, N);
  const int64_t kt = K / 64;
  if (s > kt / 32) s = (int)(kt / 32);  // at least 32 K steps per range (shorter ranges lost to the extra pass)
  if (s <= 1) return 1;
  const int64_t kts = (kt + s - 1) / s;
  return (int)((kt + kts - 1) / kts);  // no empty range
}

hipError_t launch_gemm_w4a4_group(const GemmGroup& g, bool bf16_out, hipStream_t stream) {
  const int total = g.tile_begin[g.n];
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_w4a4_group_kernel<256, 256, 2, 4>), dim3((unsigned)total), dim3(512), 0, stream, g,
                     bf16_out ? 1 : 0);
  return hipGetLastError();
}

int64_t gemm_group_tiles(int64_t M, int64_t N) { return tiles256(M, N); }

hipError_t launch_gemm_w4a4(const uint16_t* a_hat, const float* sga, const uint8_t* codes, const uint8_t* scales,
                            const float* sgw, int64_t M, int64_t N, int64_t K, void* y, bool bf16_out,
                            const uint16_t* lora_l, const uint16_t* lora_up, int rank, float* partial,
                            hipStream_t stream) {
  // 256 x 256 tiles (8 waves, 128 x 64 per wave) whenever they cover at least
  // half of the 256 CUs; otherwise 128 x 128 tiles (4 waves) for more
  // parallelism on short activations (measured on the prefill and DiT shapes),
  // split along K when the caller's workspace holds the partial sums.
  const int b = bf16_out ? 1 : 0;
  const int64_t t256 = tiles256(M, N);
  const int64_t t128 = tiles128(M, N);
  const int splits = (rank == 0 && partial) ? gemm_splits(M, N, K) : 1;
#define NVFP4_GEMM(BM, BN, WM, WN, L, S, T)                                                                      \
  hipLaunchKernelGGL((gemm_w4a4_kernel<BM, BN, WM, WN, L, S>), dim3((unsigned)(T)), dim3(WM * WN * 64), 0, stream, \
                     a_hat, sga, codes, scales, sgw, (int)M, (int)N, (int)K, y, b, lora_l, lora_up, rank, splits,   \
                     partial)
  if (t256 >= 128) {
    if (rank > 0) NVFP4_GEMM(256, 256, 2, 4, true, false, t256);
    else NVFP4_GEMM(256, 256, 2, 4, false, false, t256);
  } else {
    if (rank > 0) NVFP4_GEMM(128, 128, 2, 2, true, false, t128);
    else if (splits > 1) NVFP4_GEMM(128, 128, 2, 2, false, true, t128 * splits);
    else NVFP4_GEMM(128, 128, 2, 2, false, false, t128);
  }
#undef NVFP4_GEMM
  if (splits > 1) {
    const int64_t n = M * N;
    hipLaunchKernelGGL(gemm_splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, partial,
                       splits, n, sga, sgw, y, b);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
