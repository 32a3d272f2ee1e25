// Internal launchers of the gfx950 NVFP4 kernels (host side).  Arguments are
// validated by the C ABI layer (nvfp4_api.hip) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kMaxAmaxPartials = 512;
constexpr int kSweepCandidates = 17;  // static activation scale candidates, E4M3 448 down to 112

int amax_partial_count(int64_t n_elems, bool bf16);
// Per-workgroup partial max |x| of a tensor (amax_partial_count of them),
// without the finalize pass; the plain and the SVDQuant-smoothed input.
hipError_t launch_amax_partials_only(const void* x, bool bf16, int64_t n_elems, float* partials, hipStream_t stream);
hipError_t launch_amax_smooth_partials_only(const uint16_t* x, int64_t rows, int64_t K, const float* mult,
                                            float* partials, hipStream_t stream);
// Where an activation-quantization pass takes its tensor scale s_gA from:
// a given device fp32 (src), or this call's amax partials (partials, np),
// reduced and turned into fp32(amax / 2688) by every workgroup of the pass.
// The pass's first workgroup writes the scale to `out` (the workspace's
// s_gA, read by the product that follows).
struct ActScale {
  const float* src;
  const float* partials;
  int np;
  float* out;
};
hipError_t launch_global_scale(const void* x, bool bf16, int64_t n_elems, float* partials, float* sg_out,
                               hipStream_t stream);
hipError_t launch_global_scale_smooth(const uint16_t* x, int64_t rows, int64_t K, const float* mult,
                                      float* partials, float* sg_out, hipStream_t stream);
hipError_t launch_channel_amax(const void* x, bool bf16, int64_t rows, int64_t cols, float* amax,
                               hipStream_t stream);
hipError_t launch_running_amax(const void* x, bool bf16, int64_t n_elems, float* partials, float* amax,
                               hipStream_t stream);
int act_sweep_partial_count(int64_t n_elems);
hipError_t launch_act_scale_sweep(const uint16_t* x, int64_t n_elems, const float* amax, double* partials,
                                  double* errors, float* scale, hipStream_t stream);
hipError_t launch_quantize_absmax(const void* x, bool bf16, int64_t n_elems, const float* sg, uint8_t* codes,
                                  uint8_t* scales, hipStream_t stream);
hipError_t launch_quantize_4o6(const void* x, bool bf16, int64_t n_elems, const float* sg, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream);
hipError_t launch_quantize_mse(const void* x, bool bf16, int64_t n_elems, const float* sg, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* sg, int64_t n_elems,
                          void* out, bool bf16_out, hipStream_t stream);
// Split-K of the M > 4 decode product on short weights (partial: fp32
// [gemv_splits(M, N, K), M, N] scratch, or nullptr for no split).
int gemv_max_splits(int64_t M, int64_t N);
int gemv_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv_w4a16(const uint16_t* x, const uint8_t* codes, const uint8_t* scales, const float* sg,
                             int64_t M, int64_t N, int64_t K, void* y, bool bf16_out, float* partial,
                             hipStream_t stream);
hipError_t launch_act_quant_f16(const uint16_t* a, int64_t n_elems, ActScale sg, uint16_t* a_hat,
                                hipStream_t stream);
// K ranges the fused activation-quantization + LoRA-down pass splits each
// 16-row tile into; splits > 1 needs fp32 partials of splits * M * rank.
int lora_splits(int64_t M, int64_t K);
// mult != nullptr: SVDQuant smoothing, the pass works on bf16(x_k mult_k).
hipError_t launch_act_quant_lora(const uint16_t* a, ActScale sg, const uint16_t* down, int rank, int64_t M,
                                 int64_t K, const float* mult, uint16_t* a_hat, uint16_t* lora_l, float* partial,
                                 hipStream_t stream);
// Split-K of the W4A4 product (short activations): the most K ranges any K
// can get for an M x N output, and the count used for a given K.
int gemm_max_splits(int64_t M, int64_t N);
int gemm_splits(int64_t M, int64_t N, int64_t K);
// Several W4A4 products in one launch (256 x 256 tiles, no split, no
// low-rank branch): the activations are already quantized in each
// product's workspace.  tile_begin[i] is the first tile of product i
// (gemm_group_tiles(M, N) tiles each); tile_begin[n] the total.
constexpr int kMaxGemmGroup = 8;
struct GemmGroup {
  int n;
  int tile_begin[kMaxGemmGroup + 1];
  const uint16_t* a_hat[kMaxGemmGroup];
  const float* sga[kMaxGemmGroup];
  const uint8_t* codes[kMaxGemmGroup];
  const uint8_t* scales[kMaxGemmGroup];
  const float* sgw[kMaxGemmGroup];
  void* y[kMaxGemmGroup];
  int M[kMaxGemmGroup], N[kMaxGemmGroup], K[kMaxGemmGroup];
};
int64_t gemm_group_tiles(int64_t M, int64_t N);
hipError_t launch_gemm_w4a4_group(const GemmGroup& g, bool bf16_out, hipStream_t stream);
// partial: fp32 [gemm_splits(M, N, K), M, N] scratch, or nullptr (no split).
hipError_t launch_gemm_w4a4(const uint16_t* a_hat, const float* sga, const uint8_t* codes, const uint8_t* scales,
                            const float* sgw, int64_t M, int64_t N, int64_t K, void* y, bool bf16_out,
                            const uint16_t* lora_l, const uint16_t* lora_up, int rank, float* partial,
                            hipStream_t stream);

}  // namespace nvfp4
