"""Python binding of libnvfp4.so (include/nvfp4.h): argument marshalling only.

Every entry point takes torch tensors that live on the current HIP device and
passes raw device pointers plus torch's current stream to the C ABI; all
arithmetic runs in the library's gfx950 kernels.  A missing library raises at
first use -- there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

(OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_FLAGS, ERR_CAPTURE,
 ERR_SCRATCH) = range(11)
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
F32, BF16 = 0, 1
GLOBAL_COMPUTE, GLOBAL_GIVEN = 0, 1
OP_QUANTIZE, OP_GEMM_W4A4, OP_GEMV_W4A16, OP_GEMM_W4A4_LORA, OP_ACT_CALIBRATE, OP_GEMM_W4A4_SPLITK = (
    0, 1, 2, 3, 4, 5)
SWEEP_CANDIDATES = 17
GEMM_QUANTIZE_ACT, GEMM_REUSE_ACT = 0, 1

# name -> (restype, argtypes); mirrors include/nvfp4.h
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "nvfp4_quantize_absmax": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I, _P, _SZ, _P]),
    "nvfp4_quantize_mse": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I, _P, _SZ, _P]),
    "nvfp4_quantize_4o6": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I, _P, _SZ, _P]),
    "nvfp4_dequant": (_I, [_P, _P, _P, _I64, _I64, _P, _I, _P]),
    "nvfp4_gemv_w4a16": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "nvfp4_gemm_w4a4": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _I, _P, _SZ, _P]),
    "nvfp4_gemm_w4a4_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _I, _P]),
    "nvfp4_gemm_w4a4_group": (_I, [_P, _I64, _I, _P]),
    "nvfp4_gemm_w4a4_lora": (_I, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I, _I, _P, _SZ, _P]),
    "nvfp4_gemm_w4a4_svdq": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I, _I, _P, _SZ,
                                  _P]),
    "nvfp4_channel_amax": (_I, [_P, _I, _I64, _I64, _P, _P]),
    "nvfp4_act_amax": (_I, [_P, _I, _I64, _I64, _P, _P, _SZ, _P]),
    "nvfp4_act_scale_sweep": (_I, [_P, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_workspace_bytes": (_SZ, [_I, _I64, _I64]),
    "nvfp4_status_string": (ctypes.c_char_p, [_I]),
    "nvfp4_version": (_I, []),
}

_lib = None


class GemmProduct(ctypes.Structure):
    """nvfp4_gemm_w4a4_product of include/nvfp4.h."""
    _fields_ = [("a", _P), ("a_global", _P), ("w_codes", _P), ("w_scales", _P), ("w_global", _P), ("M", _I64),
                ("N", _I64), ("K", _I64), ("y", _P), ("flags", _I), ("workspace", _P), ("ws_bytes", _SZ)]


class NVFP4Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dit_quantization_amd.build` "
                               "(hipcc, gfx950); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status):
    return lib().nvfp4_status_string(int(status)).decode()


def workspace_bytes(op, a, b):
    return int(lib().nvfp4_workspace_bytes(int(op), int(a), int(b)))


def _check(fn, status):
    if status != OK:
        if status in (ERR_SHAPE, ERR_DTYPE, ERR_FLAGS, ERR_ALIGN, ERR_NULL):
            raise ValueError(f"{fn}: {status_string(status)} (status {status})")
        raise NVFP4Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt):
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {dt}; expected float32 or bfloat16")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")
    if torch.cuda.is_current_stream_capturing():
        # The library refuses a capturing stream too (NVFP4_ERR_CAPTURE); this
        # raises before any per-call workspace is allocated.
        raise RuntimeError("nvfp4 calls are not graph-capture safe: the current stream is being captured")


def _alloc_ws(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _quantize(fn_name, x, global_scale=None, workspace=None, out=None):
    _need_cuda(x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    if cols % 16:
        raise ValueError(f"cols={cols} is not a multiple of the 16-element block")
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        sg = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        codes, scales, sg = out
    flags = GLOBAL_COMPUTE
    if global_scale is not None:
        flags = GLOBAL_GIVEN
        sg.copy_(torch.as_tensor(global_scale, dtype=torch.float32).reshape(1))
        ws = None
    else:
        ws = workspace if workspace is not None else _alloc_ws(workspace_bytes(OP_QUANTIZE, rows, cols), dev)
    st = getattr(lib(), fn_name)(_ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(codes), _ptr(scales), _ptr(sg),
                                 flags, _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    _check(fn_name, st)
    return codes, scales, sg


def quantize_absmax(x, global_scale=None, workspace=None, out=None):
    """NVFP4 absmax quantization of a [rows, cols] fp32/bf16 GPU tensor.

    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16],
    global scale fp32 [1]).  global_scale=None computes s_g on the device."""
    return _quantize("nvfp4_quantize_absmax", x, global_scale, workspace, out)


def quantize_mse(x, global_scale=None, workspace=None, out=None):
    """NVFP4 quantization with MSE-searched block scales (same layout)."""
    return _quantize("nvfp4_quantize_mse", x, global_scale, workspace, out)


def quantize_4o6(x, global_scale=None, workspace=None, out=None):
    """NVFP4 quantization with four-over-six block scales (same layout)."""
    return _quantize("nvfp4_quantize_4o6", x, global_scale, workspace, out)


def dequant(codes, scales, global_scale, out_dtype=torch.float32, out=None):
    _need_cuda(codes, scales, global_scale)
    rows, half = codes.shape
    cols = half * 2
    if scales.shape != (rows, cols // 16):
        raise ValueError(f"scales shape {tuple(scales.shape)} does not match codes {tuple(codes.shape)}")
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=codes.device)
    st = lib().nvfp4_dequant(_ptr(codes), _ptr(scales), _ptr(global_scale), rows, cols, _ptr(out),
                             _dtype_code(out.dtype), _stream())
    _check("nvfp4_dequant", st)
    return out


def _check_weight(codes, scales, K):
    N = codes.shape[0]
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise ValueError("packed weights must be uint8 codes [N, K/2] and uint8 E4M3 scales [N, K/16]")
    if tuple(codes.shape) != (N, K // 2) or tuple(scales.shape) != (N, K // 16):
        raise ValueError(f"packed weight shapes {tuple(codes.shape)}, {tuple(scales.shape)} do not match "
                         f"K={K}: expected [N, {K // 2}] and [N, {K // 16}]")
    return N


def gemv_w4a16(x, w_codes, w_scales, w_global, out_dtype=torch.bfloat16, workspace=None, out=None, split_k=True):
    """y = x W^T for bf16 x [M, K] (M <= 16) and NVFP4 weights [N, K].

    split_k=False (with no workspace given) runs the unsplit kernel even where
    the library would split K."""
    _need_cuda(x, w_codes, w_scales, w_global)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    M, K = x.shape
    N = _check_weight(w_codes, w_scales, K)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    if workspace is not None or not split_k:
        ws = workspace
    else:
        ws = _alloc_ws(workspace_bytes(OP_GEMV_W4A16, M, N), x.device)
    st = lib().nvfp4_gemv_w4a16(_ptr(x), _ptr(w_codes), _ptr(w_scales), _ptr(w_global), M, N, K, _ptr(out),
                                _dtype_code(out.dtype), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    _check("nvfp4_gemv_w4a16", st)
    return out


def gemm_w4a4(a, w_codes, w_scales, w_global, a_global=None, out_dtype=torch.bfloat16, workspace=None,
              out=None, reuse_act=False, lora=None, smooth=None):
    """y = quant(a) W^T with per-call NVFP4 quantization of bf16 a [M, K].

    lora=(down [r, K], up [N, r]) (bf16) adds the 16-bit low-rank term
    (a down^T) up^T, fused into the same pass (r = 16, 32, ..., 128).
    smooth=[K] fp32 multipliers (with lora): the SVDQuant layer, whose input
    is bf16(a * smooth) (see svdquant.prepare).

    a_global=None computes the activation's tensor scale on the device.
    The workspace (returned contents documented in include/nvfp4.h) may be
    passed in to inspect the quantized activation; reuse_act=True multiplies
    the activation already quantized in `workspace` (same a) without
    quantizing it again."""
    _need_cuda(a, w_codes, w_scales, w_global, a_global)
    if a.dtype != torch.bfloat16 or a.dim() != 2:
        raise ValueError("a must be a 2-D bfloat16 tensor")
    M, K = a.shape
    N = _check_weight(w_codes, w_scales, K)
    if reuse_act and workspace is None:
        raise ValueError("reuse_act needs the workspace of the call that quantized the activation")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    flags = GEMM_REUSE_ACT if reuse_act else GEMM_QUANTIZE_ACT
    if smooth is not None and lora is None:
        raise ValueError("smooth needs the low-rank factors (lora=)")
    if lora is None:
        ws = workspace if workspace is not None else _alloc_ws(gemm_workspace_bytes(M, N, K), a.device)
        st = lib().nvfp4_gemm_w4a4(_ptr(a), _ptr(a_global), _ptr(w_codes), _ptr(w_scales), _ptr(w_global), M, N, K,
                                   _ptr(out), _dtype_code(out.dtype), flags, _ptr(ws), ws.numel(), _stream())
        _check("nvfp4_gemm_w4a4", st)
        return out
    down, up = lora
    _need_cuda(down, up)
    if down.dtype != torch.bfloat16 or up.dtype != torch.bfloat16 or down.dim() != 2 or up.dim() != 2:
        raise ValueError("lora = (down [r, K], up [N, r]) must be 2-D bfloat16 tensors")
    r = down.shape[0]
    if down.shape != (r, K) or up.shape != (N, r) or not down.is_contiguous() or not up.is_contiguous():
        raise ValueError("lora = (down [r, K], up [N, r]) must be contiguous with matching sizes")
    ws = workspace if workspace is not None else _alloc_ws(workspace_bytes(OP_GEMM_W4A4_LORA, M, K), a.device)
    if smooth is None:
        st = lib().nvfp4_gemm_w4a4_lora(_ptr(a), _ptr(a_global), _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                        _ptr(down), _ptr(up), r, M, N, K, _ptr(out), _dtype_code(out.dtype), flags,
                                        _ptr(ws), ws.numel(), _stream())
        _check("nvfp4_gemm_w4a4_lora", st)
        return out
    _need_cuda(smooth)
    if smooth.dtype != torch.float32 or smooth.shape != (K,):
        raise ValueError("smooth must be a float32 [K] tensor")
    st = lib().nvfp4_gemm_w4a4_svdq(_ptr(a), _ptr(a_global), _ptr(w_codes), _ptr(w_scales), _ptr(w_global),
                                    _ptr(smooth), _ptr(down), _ptr(up), r, M, N, K, _ptr(out),
                                    _dtype_code(out.dtype), flags, _ptr(ws), ws.numel(), _stream())
    _check("nvfp4_gemm_w4a4_svdq", st)
    return out


def gemm_w4a4_group(products, out_dtype=torch.bfloat16):
    """Several W4A4 products in one launch (nvfp4_gemm_w4a4_group).

    products: list of dicts with keys a (bf16 [M, K]), w (codes, scales,
    global), workspace (uint8 device tensor, at least
    workspace_bytes(OP_GEMM_W4A4, M, K)), and optionally a_global, out
    ([M, N] of out_dtype) and reuse_act (multiply what the workspace holds
    once every activation of the call is quantized).  Returns the outputs."""
    arr = (GemmProduct * max(1, len(products)))()
    outs = []
    for i, p in enumerate(products):
        a, (c, sc, g), ws = p["a"], p["w"], p["workspace"]
        ag = p.get("a_global")
        _need_cuda(a, c, sc, g, ws, ag)
        if a.dtype != torch.bfloat16 or a.dim() != 2:
            raise ValueError("a must be a 2-D bfloat16 tensor")
        M, K = a.shape
        N = _check_weight(c, sc, K)
        y = p.get("out")
        if y is None:
            y = torch.empty((M, N), dtype=out_dtype, device=a.device)
        elif y.dtype != out_dtype:
            raise ValueError("every output must have out_dtype")
        arr[i] = GemmProduct(a.data_ptr(), None if ag is None else ag.data_ptr(), c.data_ptr(), sc.data_ptr(),
                             g.data_ptr(), M, N, K, y.data_ptr(),
                             GEMM_REUSE_ACT if p.get("reuse_act") else GEMM_QUANTIZE_ACT, ws.data_ptr(), ws.numel())
        outs.append(y)
    st = lib().nvfp4_gemm_w4a4_group(arr, len(products), _dtype_code(out_dtype), _stream())
    _check("nvfp4_gemm_w4a4_group", st)
    return outs


def gemm_w4a4_noalloc(a, w_codes, w_scales, w_global, a_global=None, out_dtype=torch.bfloat16, out=None,
                      reuse_act=False):
    """The W4A4 product through nvfp4_gemm_w4a4_noalloc: the library's fixed
    64 MiB per-GPU scratch instead of a workspace (the C call allocates
    nothing; pass `out` to allocate nothing here either).  reuse_act=True
    multiplies the activation the previous call of this function on this GPU
    quantized (same a)."""
    _need_cuda(a, w_codes, w_scales, w_global, a_global)
    if a.dtype != torch.bfloat16 or a.dim() != 2:
        raise ValueError("a must be a 2-D bfloat16 tensor")
    M, K = a.shape
    N = _check_weight(w_codes, w_scales, K)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    flags = GEMM_REUSE_ACT if reuse_act else GEMM_QUANTIZE_ACT
    st = lib().nvfp4_gemm_w4a4_noalloc(_ptr(a), _ptr(a_global), _ptr(w_codes), _ptr(w_scales), _ptr(w_global), M, N,
                                       K, _ptr(out), _dtype_code(out.dtype), flags, _stream())
    _check("nvfp4_gemm_w4a4_noalloc", st)
    return out


def gemm_workspace_bytes(M, N, K, split_k=True):
    """Workspace of the plain W4A4 product; with split_k also the partial sums
    that let short activations split K."""
    return workspace_bytes(OP_GEMM_W4A4, M, K) + (workspace_bytes(OP_GEMM_W4A4_SPLITK, M, N) if split_k else 0)


def gemm_workspace_layout(M, K):
    """Byte offsets inside the W4A4 workspace: (s_gA, quantized activation fp16 [M, K])."""
    return 0, 256


def gemm_lora_l_offset(M, K):
    """Byte offset of the bf16 low-rank activation L [M, r] in the workspace of the fused LoRA product."""
    return 256 + (2 * M * K + 255) // 256 * 256


def act_amax(x, amax, workspace=None):
    """amax = max(amax, max |x|) on the device (x bf16 or fp32 [rows, cols])."""
    _need_cuda(x, amax)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    ws = workspace if workspace is not None else _alloc_ws(workspace_bytes(OP_ACT_CALIBRATE, rows, cols), x.device)
    st = lib().nvfp4_act_amax(_ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(amax), _ptr(ws), ws.numel(), _stream())
    _check("nvfp4_act_amax", st)


def act_scale_sweep(x, amax, errors, scale, workspace=None):
    """Add one bf16 calibration batch's errors for the 17 candidate static
    activation scales to `errors` (fp64 [17]) and write the current best scale."""
    _need_cuda(x, amax, errors, scale)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    if errors.dtype != torch.float64 or errors.numel() != SWEEP_CANDIDATES:
        raise ValueError("errors must be a float64 tensor of SWEEP_CANDIDATES elements")
    rows, cols = x.shape
    ws = workspace if workspace is not None else _alloc_ws(workspace_bytes(OP_ACT_CALIBRATE, rows, cols), x.device)
    st = lib().nvfp4_act_scale_sweep(_ptr(x), rows, cols, _ptr(amax), _ptr(errors), _ptr(scale), _ptr(ws),
                                     ws.numel(), _stream())
    _check("nvfp4_act_scale_sweep", st)


def calibrate_act_scale(batches):
    """Static activation tensor scale from bf16 calibration batches (all on the
    GPU): the running amax over every batch, then the FP8 candidate sweep.
    Returns (scale fp32 [1], errors fp64 [17], amax fp32 [1]) device tensors;
    pass `scale` as a_global to gemm_w4a4."""
    if not batches:
        raise ValueError("no calibration batches")
    dev = batches[0].device
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    errors = torch.zeros(SWEEP_CANDIDATES, dtype=torch.float64, device=dev)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    for b in batches:
        act_amax(b, amax)
    for b in batches:
        act_scale_sweep(b, amax, errors, scale)
    return scale, errors, amax


def channel_amax(x, amax):
    """amax[k] = max(amax[k], max_r |x[r, k]|) on the device (x bf16 or fp32 [rows, cols], amax fp32 [cols])."""
    _need_cuda(x, amax)
    if x.dim() != 2 or amax.dtype != torch.float32 or amax.shape != (x.shape[1],):
        raise ValueError("x [rows, cols] and amax float32 [cols]")
    st = lib().nvfp4_channel_amax(_ptr(x), _dtype_code(x.dtype), x.shape[0], x.shape[1], _ptr(amax), _stream())
    _check("nvfp4_channel_amax", st)
