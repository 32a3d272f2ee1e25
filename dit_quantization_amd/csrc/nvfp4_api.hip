// C ABI of the gfx950 NVFP4 library (declarations and the contract of every
// entry point: include/nvfp4.h).  This layer validates arguments without
// touching the HIP runtime, then launches the kernels on the caller's stream.
#include "../../include/nvfp4.h"

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace {

using namespace nvfp4;

constexpr int kVersion = 1 * 10000 + 5 * 100 + 0;
static_assert(kSweepCandidates == NVFP4_SWEEP_CANDIDATES, "candidate count of the activation scale sweep");

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool mul_ok(int64_t a, int64_t b) { return a >= 0 && b >= 0 && (a == 0 || b <= INT64_MAX / a); }

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t amax_ws_bytes(int64_t n, bool bf16) {
  return round256(sizeof(float) * (size_t)amax_partial_count(n, bf16));
}

// Clear a stale error from earlier unrelated work so that a launch failure
// is attributed to this call.
void clear_error() { (void)hipGetLastError(); }

int launch_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH; }

int validate_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, const uint8_t* codes,
                      const uint8_t* scales, const float* gs, int flags, const void* ws, size_t ws_bytes) {
  if (!x || !codes || !scales || !gs) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (flags & ~1) return NVFP4_ERR_FLAGS;
  if (rows < 0 || cols < 0 || !mul_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (cols % 32 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(gs, 4)) return NVFP4_ERR_ALIGN;
  if ((flags & NVFP4_GLOBAL_GIVEN) == 0) {
    if (!ws) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    if (ws_bytes < amax_ws_bytes(rows * cols, x_dtype == NVFP4_BF16)) return NVFP4_ERR_WORKSPACE;
  }
  return NVFP4_OK;
}

enum class Search { kAbsmax, kMse, kFourOverSix };

int quantize_common(Search mode, const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                    uint8_t* scales, float* gs, int flags, void* ws, size_t ws_bytes, void* stream) {
  int st = validate_quantize(x, x_dtype, rows, cols, codes, scales, gs, flags, ws, ws_bytes);
  if (st != NVFP4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  bool bf16 = x_dtype == NVFP4_BF16;
  int64_t n = rows * cols;
  clear_error();
  if ((flags & NVFP4_GLOBAL_GIVEN) == 0) {
    hipError_t e = launch_global_scale(x, bf16, n, reinterpret_cast<float*>(ws), gs, s);
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
  }
  hipError_t e = mode == Search::kAbsmax        ? launch_quantize_absmax(x, bf16, n, gs, codes, scales, s)
                 : mode == Search::kFourOverSix ? launch_quantize_4o6(x, bf16, n, gs, codes, scales, s)
                                                : launch_quantize_mse(x, bf16, n, gs, codes, scales, s);
  return launch_status(e);
}

size_t gemm_ws_bytes(int64_t M, int64_t K) {
  return 256 + round256((size_t)M * K * 2) + amax_ws_bytes(M * K, true);
}

// The low-rank variant keeps L = x lora_down^T (bf16 [M, rank <= 128]) right
// after the quantized activation and moves the amax partials behind it.
constexpr int kMaxLoraRank = 128;

size_t lora_partial_bytes(int64_t M, int64_t K) {
  const int s = K > 0 ? lora_splits(M, K) : 1;
  return s > 1 ? round256((size_t)s * M * kMaxLoraRank * 4) : 0;
}

size_t gemm_lora_ws_bytes(int64_t M, int64_t K) {
  return gemm_ws_bytes(M, K) + round256((size_t)M * kMaxLoraRank * 2) + lora_partial_bytes(M, K);
}

size_t calibrate_ws_bytes(int64_t n) {
  const size_t amax = amax_ws_bytes(n, false) > amax_ws_bytes(n, true) ? amax_ws_bytes(n, false)
                                                                        : amax_ws_bytes(n, true);
  const size_t sweep = round256(sizeof(double) * NVFP4_SWEEP_CANDIDATES * (size_t)act_sweep_partial_count(n));
  return amax > sweep ? amax : sweep;
}

int gemm_common(const void* a, const float* a_global, const uint8_t* w_codes, const uint8_t* w_scales,
                const float* w_global, const float* smooth, const void* lora_down, const void* lora_up, int rank,
                int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int flags, void* workspace, size_t ws_bytes,
                void* stream) {
  const bool reuse = (flags & NVFP4_GEMM_REUSE_ACT) != 0;
  const bool lora = rank != 0;
  if ((!a && !reuse) || !w_codes || !w_scales || !w_global || !y || !workspace) return NVFP4_ERR_NULL;
  if (lora && ((!lora_down && !reuse) || !lora_up)) return NVFP4_ERR_NULL;
  if (flags & ~1) return NVFP4_ERR_FLAGS;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || rank < 0 || !mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return NVFP4_ERR_SHAPE;
  if (K % 16 != 0) return NVFP4_ERR_SHAPE;
  // K <= 2^22: a 256-row operand panel (256 K 2 bytes) and its DMA offsets
  // stay within the 32-bit buffer ranges the kernels address.
  if (K % 64 != 0 || K == 0 || M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 22)
    return NVFP4_ERR_UNSUPPORTED;
  if (lora && (rank % 16 != 0 || rank > kMaxLoraRank)) return NVFP4_ERR_UNSUPPORTED;
  if ((!reuse && !aligned(a, 16)) || !aligned(w_codes, 16) || !aligned(w_scales, 4) || !aligned(w_global, 4) ||
      (a_global && !aligned(a_global, 4)) || !aligned(y, 16) || !aligned(workspace, 256))
    return NVFP4_ERR_ALIGN;
  if (lora && ((!reuse && !aligned(lora_down, 16)) || !aligned(lora_up, 16))) return NVFP4_ERR_ALIGN;
  if (smooth && !reuse && !aligned(smooth, 16)) return NVFP4_ERR_ALIGN;
  if (ws_bytes < (lora ? gemm_lora_ws_bytes(M, K) : gemm_ws_bytes(M, K))) return NVFP4_ERR_WORKSPACE;
  if (M == 0 || N == 0) return NVFP4_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  float* sga = reinterpret_cast<float*>(ws);
  uint16_t* a_hat = reinterpret_cast<uint16_t*>(ws + 256);
  const size_t after_a = 256 + round256((size_t)M * K * 2);
  uint16_t* lora_l = reinterpret_cast<uint16_t*>(ws + after_a);
  const size_t after_l = after_a + (lora ? round256((size_t)M * kMaxLoraRank * 2) : 0);
  float* lora_partial = reinterpret_cast<float*>(ws + after_l);
  float* partials = reinterpret_cast<float*>(ws + after_l + (lora ? lora_partial_bytes(M, K) : 0));
  clear_error();
  if (!reuse) {
    hipError_t e = hipSuccess;
    if (a_global) {
      e = hipMemcpyAsync(sga, a_global, sizeof(float), hipMemcpyDeviceToDevice, s);
    } else if (smooth) {
      e = launch_global_scale_smooth(reinterpret_cast<const uint16_t*>(a), M, K, smooth, partials, sga, s);
    } else {
      e = launch_global_scale(a, true, M * K, partials, sga, s);
    }
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
    const uint16_t* ab = reinterpret_cast<const uint16_t*>(a);
    e = lora ? launch_act_quant_lora(ab, sga, reinterpret_cast<const uint16_t*>(lora_down), rank, M, K, smooth,
                                     a_hat, lora_l, lora_partial, s)
             : launch_act_quant_f16(ab, M * K, sga, a_hat, s);
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
  }
  // Split-K partial sums (plain product on short activations) when the
  // workspace extends past the regions above by their size.
  float* split_partial = nullptr;
  if (!lora) {
    const int splits = gemm_splits(M, N, K);
    const size_t base = gemm_ws_bytes(M, K);
    if (splits > 1 && ws_bytes >= base + (size_t)splits * M * N * 4)
      split_partial = reinterpret_cast<float*>(ws + base);
  }
  return launch_status(launch_gemm_w4a4(a_hat, sga, w_codes, w_scales, w_global, M, N, K, y,
                                        y_dtype == NVFP4_BF16, lora ? lora_l : nullptr,
                                        reinterpret_cast<const uint16_t*>(lora_up), rank, split_partial, s));
}

}  // namespace

extern "C" {

int nvfp4_version(void) { return kVersion; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid shape (negative size, or cols/K not a multiple of 16)";
    case NVFP4_ERR_ALIGN: return "pointer not aligned as the kernels require";
    case NVFP4_ERR_DTYPE: return "unknown dtype";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_UNSUPPORTED: return "shape outside the supported range (K % 32, M range)";
    case NVFP4_ERR_LAUNCH: return "HIP kernel launch failed";
    case NVFP4_ERR_FLAGS: return "unknown flag bits";
    default: return "unknown status";
  }
}

size_t nvfp4_workspace_bytes(int op, int64_t a, int64_t b) {
  if (a < 0 || b < 0 || !mul_ok(a, b)) return 0;
  switch (op) {
    case NVFP4_OP_QUANTIZE: return amax_ws_bytes(a * b, false) > amax_ws_bytes(a * b, true)
                                       ? amax_ws_bytes(a * b, false) : amax_ws_bytes(a * b, true);
    case NVFP4_OP_GEMM_W4A4: return gemm_ws_bytes(a, b);
    case NVFP4_OP_GEMV_W4A16: {
      const int s = gemv_max_splits(a, b);
      return s > 1 ? round256((size_t)s * a * b * 4) : 0;
    }
    case NVFP4_OP_GEMM_W4A4_LORA: return gemm_lora_ws_bytes(a, b);
    case NVFP4_OP_ACT_CALIBRATE: return calibrate_ws_bytes(a * b);
    case NVFP4_OP_GEMM_W4A4_SPLITK: {
      const int s = gemm_max_splits(a, b);
      return s > 1 ? round256((size_t)s * a * b * 4) : 0;
    }
    default: return 0;
  }
}

int nvfp4_quantize_absmax(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                          uint8_t* scales, float* global_scale, int flags, void* workspace, size_t ws_bytes,
                          void* stream) {
  return quantize_common(Search::kAbsmax, x, x_dtype, rows, cols, codes, scales, global_scale, flags, workspace,
                         ws_bytes, stream);
}

int nvfp4_quantize_mse(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                       float* global_scale, int flags, void* workspace, size_t ws_bytes, void* stream) {
  return quantize_common(Search::kMse, x, x_dtype, rows, cols, codes, scales, global_scale, flags, workspace,
                         ws_bytes, stream);
}

int nvfp4_quantize_4o6(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                       float* global_scale, int flags, void* workspace, size_t ws_bytes, void* stream) {
  return quantize_common(Search::kFourOverSix, x, x_dtype, rows, cols, codes, scales, global_scale, flags,
                         workspace, ws_bytes, stream);
}

int nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* global_scale, int64_t rows,
                  int64_t cols, void* out, int out_dtype, void* stream) {
  if (!codes || !scales || !global_scale || !out) return NVFP4_ERR_NULL;
  if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (rows < 0 || cols < 0 || !mul_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (cols % 32 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(codes, 4) || !aligned(global_scale, 4) || !aligned(out, 16)) return NVFP4_ERR_ALIGN;
  clear_error();
  return launch_status(launch_dequant(codes, scales, global_scale, rows * cols, out, out_dtype == NVFP4_BF16,
                                      reinterpret_cast<hipStream_t>(stream)));
}

int nvfp4_gemv_w4a16(const void* x, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                     int64_t M, int64_t N, int64_t K, void* y, int y_dtype, void* workspace, size_t ws_bytes,
                     void* stream) {
  if (!x || !w_codes || !w_scales || !w_global || !y) return NVFP4_ERR_NULL;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || !mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return NVFP4_ERR_SHAPE;
  if (K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (K % 32 != 0 || M > 16 || K > (int64_t)1 << 24 || N > (int64_t)1 << 30) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(w_codes, 16) || !aligned(w_scales, 4) || !aligned(w_global, 4) ||
      !aligned(y, 4))
    return NVFP4_ERR_ALIGN;
  if (workspace && !aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (K == 0) return NVFP4_ERR_UNSUPPORTED;
  // Split-K partial sums when the workspace holds them.
  const int splits = gemv_splits(M, N, K);
  float* partial = (splits > 1 && workspace && ws_bytes >= (size_t)splits * M * N * 4)
                       ? reinterpret_cast<float*>(workspace) : nullptr;
  clear_error();
  return launch_status(launch_gemv_w4a16(reinterpret_cast<const uint16_t*>(x), w_codes, w_scales, w_global, M, N,
                                         K, y, y_dtype == NVFP4_BF16, partial,
                                         reinterpret_cast<hipStream_t>(stream)));
}

int nvfp4_gemm_w4a4(const void* a, const float* a_global, const uint8_t* w_codes, const uint8_t* w_scales,
                    const float* w_global, int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int flags,
                    void* workspace, size_t ws_bytes, void* stream) {
  return gemm_common(a, a_global, w_codes, w_scales, w_global, nullptr, nullptr, nullptr, 0, M, N, K, y, y_dtype,
                     flags, workspace, ws_bytes, stream);
}

int nvfp4_gemm_w4a4_lora(const void* a, const float* a_global, const uint8_t* w_codes, const uint8_t* w_scales,
                         const float* w_global, const void* lora_down, const void* lora_up, int64_t rank, int64_t M,
                         int64_t N, int64_t K, void* y, int y_dtype, int flags, void* workspace, size_t ws_bytes,
                         void* stream) {
  if (rank <= 0) return NVFP4_ERR_SHAPE;
  if (rank > kMaxLoraRank) return NVFP4_ERR_UNSUPPORTED;
  return gemm_common(a, a_global, w_codes, w_scales, w_global, nullptr, lora_down, lora_up, (int)rank, M, N, K, y,
                     y_dtype, flags, workspace, ws_bytes, stream);
}

int nvfp4_gemm_w4a4_svdq(const void* a, const float* a_global, const uint8_t* w_codes, const uint8_t* w_scales,
                         const float* w_global, const float* smooth, const void* lora_down, const void* lora_up,
                         int64_t rank, int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int flags,
                         void* workspace, size_t ws_bytes, void* stream) {
  if (!smooth && !(flags & NVFP4_GEMM_REUSE_ACT)) return NVFP4_ERR_NULL;
  if (rank <= 0) return NVFP4_ERR_SHAPE;
  if (rank > kMaxLoraRank) return NVFP4_ERR_UNSUPPORTED;
  return gemm_common(a, a_global, w_codes, w_scales, w_global, smooth, lora_down, lora_up, (int)rank, M, N, K, y,
                     y_dtype, flags, workspace, ws_bytes, stream);
}

int nvfp4_channel_amax(const void* x, int x_dtype, int64_t rows, int64_t cols, float* amax, void* stream) {
  if (!x || !amax) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (rows < 0 || cols < 0 || !mul_ok(rows, cols) || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (cols > (int64_t)1 << 30) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(amax, 4)) return NVFP4_ERR_ALIGN;
  clear_error();
  return launch_status(launch_channel_amax(x, x_dtype == NVFP4_BF16, rows, cols, amax,
                                           reinterpret_cast<hipStream_t>(stream)));
}

int nvfp4_act_amax(const void* x, int x_dtype, int64_t rows, int64_t cols, float* amax, void* workspace,
                   size_t ws_bytes, void* stream) {
  if (!x || !amax || !workspace) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (rows < 0 || cols < 0 || !mul_ok(rows, cols) || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(amax, 4)) return NVFP4_ERR_ALIGN;
  if (ws_bytes < calibrate_ws_bytes(rows * cols)) return NVFP4_ERR_WORKSPACE;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  clear_error();
  return launch_status(launch_running_amax(x, x_dtype == NVFP4_BF16, rows * cols, reinterpret_cast<float*>(workspace),
                                           amax, reinterpret_cast<hipStream_t>(stream)));
}

int nvfp4_act_scale_sweep(const void* x, int64_t rows, int64_t cols, const float* amax, double* errors, float* scale,
                          void* workspace, size_t ws_bytes, void* stream) {
  if (!x || !amax || !errors || !scale || !workspace) return NVFP4_ERR_NULL;
  if (rows < 0 || cols < 0 || !mul_ok(rows, cols) || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(amax, 4) || !aligned(errors, 8) || !aligned(scale, 4) || !aligned(workspace, 256))
    return NVFP4_ERR_ALIGN;
  if (ws_bytes < calibrate_ws_bytes(rows * cols)) return NVFP4_ERR_WORKSPACE;
  clear_error();
  return launch_status(launch_act_scale_sweep(reinterpret_cast<const uint16_t*>(x), rows * cols, amax,
                                              reinterpret_cast<double*>(workspace), errors, scale,
                                              reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
