/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 library:
 *   - block quantizers: nvfp4_quantize_absmax, nvfp4_quantize_mse,
 *     nvfp4_quantize_4o6 (four-over-six), and nvfp4_dequant;
 *   - W4A16 decode product: nvfp4_gemv_w4a16;
 *   - W4A4 product with per-call activation quantization: nvfp4_gemm_w4a4
 *     (nvfp4_gemm_w4a4_group for several products in one launch, and
 *     nvfp4_gemm_w4a4_noalloc, its variant on a fixed device scratch),
 *     with a fused 16-bit low-rank (LoRA) branch: nvfp4_gemm_w4a4_lora, and
 *     on an SVDQuant-smoothed input: nvfp4_gemm_w4a4_svdq;
 *   - calibration of a static activation scale: nvfp4_act_amax,
 *     nvfp4_act_scale_sweep, and per-channel ranges: nvfp4_channel_amax;
 *   - nvfp4_workspace_bytes, nvfp4_status_string, nvfp4_version.
 *
 * Format (from the pages "Tu pipeline NVFP4: meter 62 GB de modelo en 24 GB de
 * laptop", section 2 "Que es realmente NVFP4", and "NVFP4 en difusion: la
 * misma cuantizacion, un motor completamente distinto", section 2
 * "NVFP4 sin vLLM: torch._scaled_mm a mano"):
 *   - a tensor W [rows, cols] (row-major, cols = the reduction/input
 *     dimension K) is cut into 16-element blocks along cols;
 *   - each element is an E2M1 code (bit 3 sign, bits 2..1 exponent with
 *     bias 1, bit 0 mantissa; values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 *     negatives), packed two per byte: codes[r, i] = code(W[r, 2i]) |
 *     code(W[r, 2i+1]) << 4  (low nibble = even column);
 *   - each block has one FP8 E4M3 ("fn": bias 7, max 448, no infinities)
 *     scale byte: scales[r, j] for elements j*16 .. j*16+15 of row r;
 *   - the tensor has one fp32 second-level scale s_g;
 *   - reconstruction: W^ = q * s_b * s_g.
 * Encoding rules (the pages leave these open; this library fixes them):
 *   - s_g = fp32(amax(|W|) / 2688), 2688 = 6 * 448 (1.0 for an all-zero
 *     tensor), or a caller-given value;
 *   - absmax block scale s_b = nearest E4M3 to amax_block / (6 s_g), exact
 *     ties to the even code, saturating at 448;
 *   - MSE block scale: the candidate with the least squared reconstruction
 *     error among the E4M3 values c > 0 with a/2 <= c <= min(2a, 448)
 *     (a = amax_block / (6 s_g)) plus the absmax scale; error summed in fp64,
 *     element order, one rounding per operation; ties keep the smaller c;
 *   - element code = nearest E2M1 value to W / (s_b s_g), exact ties to the
 *     even code, saturating at 6; zero is always code 0 (never -0); all
 *     codes are 0 when s_b = 0.
 * Codes and scale bytes are bit-exact functions of the input.
 *
 * Conventions for every call:
 *   - all pointers are DEVICE pointers (memory of the current HIP device),
 *     row-major and contiguous; `stream` is a hipStream_t (NULL = default);
 *   - calls are asynchronous on `stream`; the library never allocates,
 *     frees or synchronizes the host in a call;
 *   - the caller owns every buffer; inputs are never modified;
 *   - arguments are validated before any launch; on error nothing is
 *     launched and the status is returned;
 *   - a product or dequantization with an empty output (M = 0 or N = 0;
 *     rows = 0 or cols = 0) launches nothing and reads none of its
 *     pointers, which may then be NULL (its sizes, dtypes and flags are
 *     still checked); a quantizer given an empty tensor takes NULL x, codes
 *     and scales (with NVFP4_GLOBAL_COMPUTE it still writes s_g = 1.0, so
 *     global_scale and the workspace are needed); the calibration calls
 *     always need their pointers;
 *   - the fast path requires cols (K) % 32 == 0 and 16-byte aligned
 *     pointers (4-byte for scales, global scale and 1-row outputs);
 *     otherwise NVFP4_ERR_UNSUPPORTED / NVFP4_ERR_ALIGN is returned;
 *   - non-finite inputs are a caller error: the outputs are unspecified;
 *   - calls are NOT graph-capture safe: after the arguments are validated,
 *     every call that would launch asks the runtime whether `stream` is
 *     being captured and, if so, returns NVFP4_ERR_CAPTURE without
 *     launching (NVFP4_ERR_LAUNCH if the runtime cannot tell).
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,       /* negative size, or cols/K not a multiple of 16 */
  NVFP4_ERR_ALIGN = 3,       /* pointer alignment below what the kernels load */
  NVFP4_ERR_DTYPE = 4,       /* unknown dtype code */
  NVFP4_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than nvfp4_workspace_bytes */
  NVFP4_ERR_UNSUPPORTED = 6, /* valid NVFP4 shape outside the kernels' range (K % 32, M > 16, ...) */
  NVFP4_ERR_LAUNCH = 7,      /* the HIP runtime reported an error at launch */
  NVFP4_ERR_FLAGS = 8,       /* unknown flag bits */
  NVFP4_ERR_CAPTURE = 9,     /* `stream` is being captured into a HIP graph (calls are not capture-safe) */
  NVFP4_ERR_SCRATCH = 10     /* nvfp4_gemm_w4a4_noalloc: the call needs more than its fixed scratch */
} nvfp4_status;

/* Size of the fixed per-GPU device scratch of nvfp4_gemm_w4a4_noalloc. */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 * 1024 * 1024)

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;

/* flags for the quantizers (bit 0) */
enum { NVFP4_GLOBAL_COMPUTE = 0, NVFP4_GLOBAL_GIVEN = 1 };

/* flags for nvfp4_gemm_w4a4 (bit 0) */
enum { NVFP4_GEMM_QUANTIZE_ACT = 0, NVFP4_GEMM_REUSE_ACT = 1 };

/* operation ids for nvfp4_workspace_bytes */
enum {
  NVFP4_OP_QUANTIZE = 0,
  NVFP4_OP_GEMM_W4A4 = 1,
  NVFP4_OP_GEMV_W4A16 = 2,
  NVFP4_OP_GEMM_W4A4_LORA = 3,
  NVFP4_OP_ACT_CALIBRATE = 4,
  NVFP4_OP_GEMM_W4A4_SPLITK = 5
};

/* number of candidate scales of nvfp4_act_scale_sweep */
enum { NVFP4_SWEEP_CANDIDATES = 17 };

/*
 * nvfp4_quantize_absmax -- NVFP4 encoding with absmax block scales.
 * ("Tu pipeline NVFP4 ...", section 2: absmax sets the block scale so that
 * the largest magnitude lands on the top grid value, s = max|W_k| / 6.)
 *   x            [rows, cols] input, dtype x_dtype (NVFP4_F32 or NVFP4_BF16)
 *   codes        [rows, cols/2] uint8 output (two E2M1 codes per byte)
 *   scales       [rows, cols/16] uint8 output (E4M3 bytes, 0x00..0x7E)
 *   global_scale one fp32 on the device: written (s_g) with
 *                NVFP4_GLOBAL_COMPUTE, read with NVFP4_GLOBAL_GIVEN
 *                (must then be finite and > 0)
 *   workspace    device scratch of >= nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE,
 *                rows, cols) bytes (may be NULL with NVFP4_GLOBAL_GIVEN);
 *                holds per-workgroup amax partials; contents on return are
 *                unspecified
 * rows == 0 is a valid no-op (s_g = 1.0 is still written in COMPUTE mode).
 */
int nvfp4_quantize_absmax(const void* x, int x_dtype, int64_t rows, int64_t cols,
                          uint8_t* codes, uint8_t* scales, float* global_scale,
                          int flags, void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_quantize_mse -- NVFP4 encoding with MSE-searched block scales.
 * ("Tu pipeline NVFP4 ...", section 2, box "Derivacion del objetivo de
 * optimizacion MSE vs Absmax": the block scale is the argmin over s_b of
 * sum_k (W_k - s_b s_g Q(W_k / (s_b s_g)))^2; the algorithm table: several
 * candidate scales are tried and the one with the least block
 * reconstruction error is kept.)  Same arguments and layout as
 * nvfp4_quantize_absmax.  Candidates: the absmax scale plus every positive
 * E4M3 value c with a/2 <= c <= min(2a, 448), a = max|W| / (6 s_g).  Error:
 * d_k = |W_k| - c s_g |q_k| rounded once in fp64, E = fp64 sum of the
 * rounded squares in element order; candidates in ascending order, replaced
 * only on a strictly smaller error.  The chosen block error is never larger
 * than the absmax scale's error.
 */
int nvfp4_quantize_mse(const void* x, int x_dtype, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales, float* global_scale,
                       int flags, void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_quantize_4o6 -- NVFP4 encoding with four-over-six block scales
 * ("Tu pipeline NVFP4 ...", section 2, algorithm table: every block picks
 * between two largest representable values, 4 or 6, whichever reconstructs
 * it with the smaller error).  Same arguments and layout as
 * nvfp4_quantize_absmax.  Candidates: the nearest E4M3 values to
 * max|W| / (6 s_g) (the absmax scale) and to max|W| / (4 s_g); the error
 * and tie rule are nvfp4_quantize_mse's (a tie keeps the absmax scale).
 */
int nvfp4_quantize_4o6(const void* x, int x_dtype, int64_t rows, int64_t cols,
                       uint8_t* codes, uint8_t* scales, float* global_scale,
                       int flags, void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_dequant -- W^ = q * s_b * s_g ("Tu pipeline NVFP4 ...", section 2,
 * hierarchical reconstruction).  q * s_b is exact in fp32; the product with
 * s_g is rounded once to fp32 (out_dtype NVFP4_F32) and that fp32 value is
 * rounded to nearest-even bf16 for NVFP4_BF16.
 *   codes [rows, cols/2], scales [rows, cols/16], global_scale: 1 device fp32
 *   out   [rows, cols] of out_dtype
 */
int nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                  int64_t rows, int64_t cols, void* out, int out_dtype, void* stream);

/*
 * nvfp4_gemv_w4a16 -- weight-only decode product y = x W^T with NVFP4
 * weights and bf16 activations ("Tu pipeline NVFP4 ...", section 2:
 * W4A16 keeps the weights in 4 bits and unpacks them to 16 bits for the
 * matmul; decoding reads every weight once per token and is bound by
 * memory bandwidth).
 *   y[m, n] = s_gW * sum_k x[m, k] * q[n, k] * s_b[n, k/16]
 *   x        [M, K] bf16;  w_codes [N, K/2];  w_scales [N, K/16];
 *   w_global 1 device fp32; y [M, N] of y_dtype (NVFP4_BF16 or NVFP4_F32)
 *   workspace optional: with at least nvfp4_workspace_bytes(
 *            NVFP4_OP_GEMV_W4A16, M, N) bytes (256-byte aligned), products
 *            with M > 4, N < 8192 and K >= 8192 cut K into up to 8 ranges
 *            whose fp32 sums are added in range order (reproducible; they may
 *            differ from the unsplit sum by fp32 rounding); NULL or a smaller
 *            workspace: no split (the size is 0 for shapes never split)
 *   0 <= M <= 16 (the decode batch; M = 0 or N = 0 is a no-op); K % 32 == 0
 *   and 0 < K <= 2^24, otherwise NVFP4_ERR_UNSUPPORTED.  fp32 accumulation,
 *   fp32 epilogue (x s_gW), round-to-nearest-even bf16 output.
 */
int nvfp4_gemv_w4a16(const void* x, const uint8_t* w_codes, const uint8_t* w_scales,
                     const float* w_global, int64_t M, int64_t N, int64_t K,
                     void* y, int y_dtype, void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_gemm_w4a4 -- y = A^ W^^T with the activation quantized to NVFP4 on
 * every call ("NVFP4 en difusion ...", section 2: out = (A s_a)(B s_b)^T with
 * bf16 output; the activation is quantized dynamically, 16-element block by
 * 16-element block, on each call, with the same absmax criterion).
 *   a        [M, K] bf16 activations
 *   a_global NULL: s_gA = fp32(amax(|A|) / 2688) computed on the device;
 *            otherwise a device fp32 used as s_gA (a static activation scale)
 *   w_codes [N, K/2], w_scales [N, K/16], w_global: the NVFP4 weight
 *   y        [M, N] of y_dtype (NVFP4_BF16 or NVFP4_F32)
 *   K % 64 == 0 (one K step of the kernel; all configured shapes qualify)
 *   and K <= 2^22 (32-bit addressing of a 256-row operand panel),
 *   otherwise NVFP4_ERR_UNSUPPORTED; M, N <= 2^30 and at most 2^27 output
 *   tiles of 128 x 128 (M N up to about 2^41), else NVFP4_ERR_UNSUPPORTED.
 *   workspace >= nvfp4_workspace_bytes(NVFP4_OP_GEMM_W4A4, M, K) bytes,
 *            256-byte aligned.  On return it holds, at fixed offsets:
 *              [0, 4)       s_gA (fp32)
 *              [256, 256 + 2*M*K)  A^ / s_gA = q_a * s_a as fp16 [M, K]
 *                           (exact: <= 6 significant bits, magnitudes in
 *                           [2^-10, 2688]), i.e. the quantized activation
 *              after that   amax partials (unspecified)
 *   flags    NVFP4_GEMM_QUANTIZE_ACT: quantize `a` into the workspace, then
 *            multiply; NVFP4_GEMM_REUSE_ACT: the workspace already holds the
 *            quantized activation of the same [M, K] input from an earlier
 *            call on this stream (several weights sharing one input, e.g.
 *            q/k/v or gate/up projections): only the product runs, and `a`
 *            and `a_global` are not read.
 *   y[m, n] = round(fp32(s_gA * s_gW) * sum_k (q_a s_a)[m,k] (q_w s_w)[n,k])
 *   with the products exact and the sum accumulated in fp32.
 *   Split-K: when the output has few tiles (short activations) and the
 *   workspace is at least nvfp4_workspace_bytes(NVFP4_OP_GEMM_W4A4, M, K) +
 *   nvfp4_workspace_bytes(NVFP4_OP_GEMM_W4A4_SPLITK, M, N) bytes, K is cut
 *   into up to 8 ranges whose fp32 sums are added in range order (a fixed
 *   order, so results are reproducible; they may differ from the unsplit sum
 *   by fp32 rounding).  With a smaller workspace the product is not split.
 */
int nvfp4_gemm_w4a4(const void* a, const float* a_global, const uint8_t* w_codes,
                    const uint8_t* w_scales, const float* w_global,
                    int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int flags,
                    void* workspace, size_t ws_bytes, void* stream);

/* One product of nvfp4_gemm_w4a4_group: the arguments of one
 * nvfp4_gemm_w4a4 call (y_dtype and stream are the group's). */
typedef struct {
  const void* a;              /* [M, K] bf16 (not read with NVFP4_GEMM_REUSE_ACT) */
  const float* a_global;      /* NULL: dynamic s_gA; else a device fp32 (static s_gA) */
  const uint8_t* w_codes;     /* [N, K/2] */
  const uint8_t* w_scales;    /* [N, K/16] */
  const float* w_global;      /* one device fp32 */
  int64_t M, N, K;
  void* y;                    /* [M, N] of the group's y_dtype */
  int flags;                  /* NVFP4_GEMM_QUANTIZE_ACT or NVFP4_GEMM_REUSE_ACT */
  void* workspace;            /* >= nvfp4_workspace_bytes(NVFP4_OP_GEMM_W4A4, M, K), 256-byte aligned */
  size_t ws_bytes;
} nvfp4_gemm_w4a4_product;

/*
 * nvfp4_gemm_w4a4_group -- several independent W4A4 products in one launch
 * per 8 products ("NVFP4 en difusion ...", section 1: a double-stream DiT
 * block sends image and text tokens through separate weights, so each of its
 * layers is one product per stream; section 2: the per-call activation
 * quantization and out = (A s_a)(B s_b)^T of nvfp4_gemm_w4a4).  Each product
 * gives the same result bit for bit as nvfp4_gemm_w4a4 would without split-K
 * partials: 256 x 256 tiles of all the products share one grid, so a phase
 * whose products each leave part of the chip idle fills it.
 *   products  host array of n descriptors, read during the call only;
 *             n >= 0 (NVFP4_ERR_SHAPE if negative, NVFP4_ERR_NULL for NULL
 *             with n > 0); every descriptor is checked as nvfp4_gemm_w4a4
 *             checks its arguments, before anything is launched
 *   y_dtype   NVFP4_BF16 or NVFP4_F32, for every product
 * Order: every product with NVFP4_GEMM_QUANTIZE_ACT first quantizes its
 * activation into its workspace (in array order), then all the products run;
 * a product with NVFP4_GEMM_REUSE_ACT multiplies what its workspace holds at
 * that point, e.g. the activation another product of the same call quantized
 * into the same workspace (q, k and v sharing one input).  Two products that
 * quantize must not share a workspace, and no output may overlap an input or
 * workspace of the call.
 */
int nvfp4_gemm_w4a4_group(const nvfp4_gemm_w4a4_product* products, int64_t n, int y_dtype, void* stream);

/*
 * nvfp4_gemm_w4a4_noalloc -- nvfp4_gemm_w4a4 for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * allocation): the same product, kernels and results, with no workspace
 * argument.  Its scratch is a fixed array of NVFP4_NOALLOC_SCRATCH_BYTES
 * (64 MiB) in device memory that the library holds on every GPU it runs on
 * until the process ends; the call itself allocates and frees nothing.
 *   a, a_global, w_codes, w_scales, w_global, M, N, K, y, y_dtype: as
 *            nvfp4_gemm_w4a4
 *   The call needs nvfp4_workspace_bytes(NVFP4_OP_GEMM_W4A4, M, K) bytes of
 *   scratch (about 2 M K): larger calls return NVFP4_ERR_SCRATCH before
 *   anything is launched.  Short activations split K (as nvfp4_gemm_w4a4
 *   with the split-K extra) when the partial sums fit in the rest of the
 *   scratch.
 *   flags    NVFP4_GEMM_QUANTIZE_ACT, or NVFP4_GEMM_REUSE_ACT: the scratch
 *            still holds the quantized activation of the same [M, K] input
 *            from the previous call of this function on this GPU
 *            (several weights sharing one input).
 * Every call on a GPU uses that GPU's one scratch array and leaves its
 * contents behind for the next (laid out as nvfp4_gemm_w4a4's workspace;
 * no part of it has to start at zero: each call writes what it reads).
 * Calls that may overlap on one GPU (different streams, or host threads
 * without ordering) race on it; the caller serializes them, e.g. by issuing
 * them on one stream.  `stream` must belong to the current device (the
 * scratch used is that device's): otherwise NVFP4_ERR_UNSUPPORTED.
 */
int nvfp4_gemm_w4a4_noalloc(const void* a, const float* a_global, const uint8_t* w_codes,
                            const uint8_t* w_scales, const float* w_global,
                            int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int flags,
                            void* stream);

/*
 * nvfp4_gemm_w4a4_lora -- the W4A4 product plus a 16-bit low-rank branch,
 * y = A^ W^^T + (A lora_down^T) lora_up^T ("NVFP4 en difusion ...",
 * section 3: a LoRA cannot be merged into weights already rounded to 4 bits,
 * so the layer evaluates W_4bit x + B (A x) at run time, the low-rank term
 * in 16 bits, in the same pass that quantizes the activation).
 *   a, a_global, w_codes, w_scales, w_global, M, N, K, y, y_dtype:
 *            as nvfp4_gemm_w4a4 (the low-rank term reads the bf16 `a`, not
 *            its quantized copy)
 *   lora_down [rank, K] bf16 (the LoRA "A"), 16-byte aligned
 *   lora_up   [N, rank] bf16 (the LoRA "B"; fold any LoRA scale into it),
 *            16-byte aligned
 *   rank     16, 32, ..., 128 (NVFP4_ERR_UNSUPPORTED otherwise, and for
 *            K > 2^22; rank <= 0 is NVFP4_ERR_SHAPE)
 *   workspace >= nvfp4_workspace_bytes(NVFP4_OP_GEMM_W4A4_LORA, M, K)
 *            bytes, 256-byte aligned, laid out as nvfp4_gemm_w4a4's, with
 *            L = bf16(A lora_down^T) [M, rank] (row stride rank) starting
 *            at byte 256 + round_up(2 M K, 256)
 *   flags    NVFP4_GEMM_REUSE_ACT reuses both the quantized activation and
 *            L: it needs an earlier call of this function on the same
 *            workspace with the same a, a_global, lora_down and rank
 *            (lora_down is then not read)
 *   L[m, j] = bf16(sum_k a[m,k] lora_down[j,k]), fp32 accumulation;
 *   y[m, n] = round(fp32(s_gA s_gW) * P[m, n] + sum_j L[m,j] lora_up[n,j])
 *   with P the W4A4 sum above and the low-rank sum accumulated in fp32
 *   onto the scaled product.
 */
int nvfp4_gemm_w4a4_lora(const void* a, const float* a_global, const uint8_t* w_codes,
                         const uint8_t* w_scales, const float* w_global,
                         const void* lora_down, const void* lora_up, int64_t rank,
                         int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int flags,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_gemm_w4a4_svdq -- the low-rank W4A4 product on an SVDQuant-smoothed
 * activation ("NVFP4 en difusion ...", section 3: SVDQuant moves activation
 * outliers into the weights by scaling channel by channel, then keeps a
 * 16-bit low-rank SVD component of the scaled weights beside the 4-bit
 * residual; that component has a LoRA's shape and runs in the same fused
 * pass).  The layer's input becomes x^[m,k] = bf16(fp32(a[m,k] * smooth[k]))
 * (round to nearest even twice), and then
 *   y = W4A4(x^, R^) + bf16(x^ lora_down^T) lora_up^T
 * exactly as nvfp4_gemm_w4a4_lora computes it on x^: s_gA is computed from
 * x^ (or given: a scale calibrated on x^), and the workspace holds the
 * quantized x^ and L.
 *   smooth   [K] device fp32 multipliers 1/lambda_k (16-byte aligned); the
 *            weights were prepared as W' = W diag(lambda), split into the
 *            rank-r factors (lora_up [N, r] lora_down [r, K], bf16) and the
 *            residual R = W' - lora_up lora_down, quantized to w_codes,
 *            w_scales, w_global.  A user LoRA (A, B) can ride along as extra
 *            rank: down rows A diag(lambda), up columns B.
 *   everything else as nvfp4_gemm_w4a4_lora; smooth is not read with
 *   NVFP4_GEMM_REUSE_ACT (the earlier call's x^ is reused).
 */
int nvfp4_gemm_w4a4_svdq(const void* a, const float* a_global, const uint8_t* w_codes,
                         const uint8_t* w_scales, const float* w_global, const float* smooth,
                         const void* lora_down, const void* lora_up, int64_t rank,
                         int64_t M, int64_t N, int64_t K, void* y, int y_dtype, int flags,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_channel_amax -- per-channel running range of calibration
 * activations (or of a weight's input columns), the statistic SVDQuant's
 * smoothing needs: amax[k] = max(amax[k], max_r |x[r, k]|).
 *   x      [rows, cols] of x_dtype (NVFP4_BF16 or NVFP4_F32), 16-byte aligned
 *   amax   [cols] device fp32, read and written; zero it before the first
 *          batch.  The result does not depend on the order of the updates.
 *   cols % 16 == 0 (NVFP4_ERR_SHAPE otherwise); rows == 0 is a no-op.
 */
int nvfp4_channel_amax(const void* x, int x_dtype, int64_t rows, int64_t cols, float* amax,
                       void* stream);

/*
 * nvfp4_act_amax -- running range of calibration activations:
 * *amax = max(*amax, max |x|).  ("Tu pipeline NVFP4 ...", section 1,
 * question 3: activation scales come from calibration, which records the
 * ranges of real activations.)
 *   x       [rows, cols] of x_dtype (NVFP4_BF16 or NVFP4_F32), 16-byte aligned
 *   amax    one device fp32, read and written; set it to 0 before the first
 *           batch
 *   workspace >= nvfp4_workspace_bytes(NVFP4_OP_ACT_CALIBRATE, rows, cols)
 *   cols % 16 == 0 (NVFP4_ERR_SHAPE otherwise); rows == 0 is a no-op.
 */
int nvfp4_act_amax(const void* x, int x_dtype, int64_t rows, int64_t cols, float* amax,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * nvfp4_act_scale_sweep -- FP8 candidate sweep for a static activation
 * tensor scale s_gA ("Tu pipeline NVFP4 ...", section 2, project box: the MSE
 * calibration also sweeps candidate activation scales in FP8).  Candidate
 * c = 0 .. NVFP4_SWEEP_CANDIDATES-1 puts the block scale of the calibration
 * set's largest block on the E4M3 value v_c = 448, 416, ..., 120, 112 (E4M3
 * byte 0x7E - c): s_c = fp32(amax / (6 v_c)), and s_c = 1 when amax == 0;
 * c = 0 is the dynamic rule's s_gA.  For one batch of calibration
 * activations:
 *   errors[c] += sum over the batch's 16-element blocks of the squared error
 *                of the block after the W4A4 activation quantization (absmax
 *                block scales) with s_gA = s_c, d = |x| - s_b s_c |q| rounded
 *                once and squared in fp64;
 *   *scale     = s_c of the smallest errors[c] so far (ties: lower c).
 *   x       [rows, cols] bf16, 16-byte aligned; cols % 16 == 0
 *   amax    one device fp32: the running range over ALL calibration batches
 *           (nvfp4_act_amax over every batch first)
 *   errors  NVFP4_SWEEP_CANDIDATES device doubles, 8-byte aligned; set them
 *           to 0 before the first batch; batches accumulate in call order
 *           (the sums inside one call are in a fixed order, so results are
 *           reproducible)
 *   scale   one device fp32, written: pass it as a_global to the W4A4
 *           products, which then quantize activations in one pass
 *   workspace >= nvfp4_workspace_bytes(NVFP4_OP_ACT_CALIBRATE, rows, cols)
 * rows == 0 adds nothing but still writes *scale.
 */
int nvfp4_act_scale_sweep(const void* x, int64_t rows, int64_t cols, const float* amax,
                          double* errors, float* scale, void* workspace, size_t ws_bytes,
                          void* stream);

/* Workspace size in bytes for an operation: NVFP4_OP_QUANTIZE and
 * NVFP4_OP_ACT_CALIBRATE with (rows, cols), NVFP4_OP_GEMM_W4A4 and
 * NVFP4_OP_GEMM_W4A4_LORA with (M, K), NVFP4_OP_GEMV_W4A16 and
 * NVFP4_OP_GEMM_W4A4_SPLITK (the optional split-K extra of nvfp4_gemm_w4a4,
 * 0 when that output is never split) with (M, N); 0 for an unknown op or
 * negative sizes. */
size_t nvfp4_workspace_bytes(int op, int64_t rows_or_m, int64_t cols_or_k);

/* Static, NUL-terminated description of a status code. */
const char* nvfp4_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int nvfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
