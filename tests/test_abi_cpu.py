"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

from dit_quantization_amd import nvfp4 as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

A16 = 0x10000          # fake, aligned, non-null addresses: validation never dereferences
A4 = 0x10004
BIG = 1 << 40


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = nv.lib()
    names = header_functions()
    assert len(names) == 16, names
    for n in names:
        assert hasattr(L, n), n
        assert n in nv.SIGNATURES, n


def test_status_strings_and_version():
    assert nv.lib().nvfp4_version() == 10801
    for s in range(11):
        assert nv.status_string(s) and nv.status_string(s) != "unknown status"
    assert nv.status_string(99) == "unknown status"


def test_workspace_sizes():
    assert nv.workspace_bytes(nv.OP_QUANTIZE, 4096, 4096) >= 4 * 1 and nv.workspace_bytes(nv.OP_QUANTIZE, 4096, 4096) % 256 == 0
    g = nv.workspace_bytes(nv.OP_GEMM_W4A4, 4096, 4096)
    assert g >= 256 + 2 * 4096 * 4096
    assert nv.workspace_bytes(nv.OP_GEMV_W4A16, 16, 4096) == 4 * 16 * 4096 * 4   # optional split-K partials
    assert nv.workspace_bytes(nv.OP_GEMV_W4A16, 4, 4096) == 0
    assert nv.workspace_bytes(nv.OP_GEMV_W4A16, 16, 14336) == 0
    # the low-rank variant adds L (bf16 [M, 128] at most) after the quantized activation
    # (and, for short activations, fp32 partial sums of the split down projection)
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4_LORA, 4096, 4096) >= g + 2 * 4096 * 128
    g16 = nv.workspace_bytes(nv.OP_GEMM_W4A4, 16384, 1024)
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4_LORA, 16384, 1024) == g16 + 2 * 16384 * 128
    assert nv.gemm_lora_l_offset(100, 64) == 256 + 12800
    assert nv.workspace_bytes(99, 1, 1) == 0
    # split-K partials: only for outputs with few tiles (at most 8 ranges)
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4_SPLITK, 4096, 14336) == 0
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4_SPLITK, 512, 12288) == 0
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4_SPLITK, 512, 3072) == 4 * 512 * 3072 * 4
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4_SPLITK, 1, 64) == 8 * 64 * 4
    assert nv.workspace_bytes(nv.OP_QUANTIZE, -1, 16) == 0


def q(fn, x=A16, dt=nv.F32, rows=4, cols=64, codes=A16, scales=A16, gs=A4, flags=nv.GLOBAL_GIVEN, ws=None, wsb=0):
    return getattr(nv.lib(), fn)(x, dt, rows, cols, codes, scales, gs, flags, ws, wsb, None)


@pytest.mark.parametrize("fn", ["nvfp4_quantize_absmax", "nvfp4_quantize_mse", "nvfp4_quantize_4o6"])
def test_quantize_validation(fn):
    assert q(fn, x=None) == nv.ERR_NULL
    assert q(fn, codes=None) == nv.ERR_NULL
    assert q(fn, gs=None) == nv.ERR_NULL
    assert q(fn, dt=7) == nv.ERR_DTYPE
    assert q(fn, flags=4) == nv.ERR_FLAGS
    assert q(fn, rows=-1) == nv.ERR_SHAPE
    assert q(fn, cols=24) == nv.ERR_SHAPE          # not a multiple of the 16-element block
    assert q(fn, cols=48) == nv.ERR_UNSUPPORTED    # a valid block count, off the K % 32 fast path
    assert q(fn, rows=BIG, cols=BIG) == nv.ERR_SHAPE
    assert q(fn, x=A16 + 4) == nv.ERR_ALIGN
    assert q(fn, codes=A16 + 2) == nv.ERR_ALIGN
    assert q(fn, flags=nv.GLOBAL_COMPUTE, ws=None) == nv.ERR_WORKSPACE
    assert q(fn, flags=nv.GLOBAL_COMPUTE, ws=A16, wsb=4) == nv.ERR_WORKSPACE


def test_dequant_validation():
    L = nv.lib()
    assert L.nvfp4_dequant(None, A16, A4, 4, 64, A16, nv.F32, None) == nv.ERR_NULL
    assert L.nvfp4_dequant(A16, A16, A4, 4, 64, A16, 3, None) == nv.ERR_DTYPE
    assert L.nvfp4_dequant(A16, A16, A4, 4, 40, A16, nv.F32, None) == nv.ERR_SHAPE
    assert L.nvfp4_dequant(A16, A16, A4, 4, 48, A16, nv.F32, None) == nv.ERR_UNSUPPORTED
    assert L.nvfp4_dequant(A16, A16, A4, 4, 64, A16 + 8, nv.F32, None) == nv.ERR_ALIGN


def test_gemv_validation():
    L = nv.lib()
    f = L.nvfp4_gemv_w4a16
    assert f(None, A16, A16, A4, 1, 64, 64, A16, nv.BF16, None, 0, None) == nv.ERR_NULL
    assert f(A16, A16, A16, A4, 1, 64, 64, A16, 5, None, 0, None) == nv.ERR_DTYPE
    assert f(A16, A16, A16, A4, 1, 64, 40, A16, nv.BF16, None, 0, None) == nv.ERR_SHAPE
    assert f(A16, A16, A16, A4, 17, 64, 64, A16, nv.BF16, None, 0, None) == nv.ERR_UNSUPPORTED
    assert f(A16, A16, A16, A4, 1, 64, 48, A16, nv.BF16, None, 0, None) == nv.ERR_UNSUPPORTED
    assert f(A16 + 2, A16, A16, A4, 1, 64, 64, A16, nv.BF16, None, 0, None) == nv.ERR_ALIGN
    assert f(A16, A16, A16, A4, 1, 64, (1 << 24) + 32, A16, nv.BF16, None, 0, None) == nv.ERR_UNSUPPORTED
    assert f(A16, A16, A16, A4, 0, 64, 64, A16, nv.BF16, None, 0, None) == nv.OK      # empty: no launch
    assert f(A16, A16, A16, A4, 8, 64, 64, A16, nv.BF16, A16 + 16, 1 << 20, None) == nv.ERR_ALIGN


def test_gemm_validation():
    L = nv.lib()
    f = L.nvfp4_gemm_w4a4
    W = 1 << 30
    Q, R = nv.GEMM_QUANTIZE_ACT, nv.GEMM_REUSE_ACT
    assert f(None, None, A16, A16, A4, 64, 64, 64, A16, nv.BF16, Q, A16, W, None) == nv.ERR_NULL
    assert f(A16, None, A16, A16, A4, 64, 64, 64, A16, nv.BF16, Q, None, W, None) == nv.ERR_NULL
    assert f(A16, None, A16, A16, A4, 64, 64, 64, A16, 9, Q, A16, W, None) == nv.ERR_DTYPE
    assert f(A16, None, A16, A16, A4, 64, 64, 64, A16, nv.BF16, 6, A16, W, None) == nv.ERR_FLAGS
    assert f(A16, None, A16, A16, A4, 64, 64, 40, A16, nv.BF16, Q, A16, W, None) == nv.ERR_SHAPE
    assert f(A16, None, A16, A16, A4, 64, 64, 96, A16, nv.BF16, Q, A16, W, None) == nv.ERR_UNSUPPORTED
    # K beyond 2^22 would overflow the 32-bit addressing of a 256-row panel
    assert f(A16, None, A16, A16, A4, 64, 64, (1 << 22) + 64, A16, nv.BF16, Q, A16, 1 << 40, None) == nv.ERR_UNSUPPORTED
    assert f(A16, None, A16, A16, A4, 64, 64, 64, A16, nv.BF16, Q, A16 + 16, W, None) == nv.ERR_ALIGN
    assert f(A16, None, A16, A16, A4, 64, 64, 64, A16, nv.BF16, Q, A16, 16, None) == nv.ERR_WORKSPACE
    assert f(A16, None, A16, A16, A4, 0, 64, 64, A16, nv.BF16, Q, A16, W, None) == nv.OK
    assert f(None, None, A16, A16, A4, 0, 64, 64, A16, nv.BF16, R, A16, W, None) == nv.OK  # reuse: a unused


def test_gemm_lora_validation():
    L = nv.lib()
    f = L.nvfp4_gemm_w4a4_lora
    W = 1 << 30
    Q, R = nv.GEMM_QUANTIZE_ACT, nv.GEMM_REUSE_ACT

    def call(a=A16, down=A16, up=A16, rank=32, M=64, N=64, K=64, flags=Q, ws=A16, wsb=W):
        return f(a, None, A16, A16, A4, down, up, rank, M, N, K, A16, nv.BF16, flags, ws, wsb, None)

    assert call(down=None) == nv.ERR_NULL
    assert call(up=None) == nv.ERR_NULL
    assert call(down=None, up=A16, flags=R, M=0) == nv.OK        # reuse: lora_down unused
    assert call(rank=0) == nv.ERR_SHAPE
    assert call(rank=-16) == nv.ERR_SHAPE
    assert call(rank=8) == nv.ERR_UNSUPPORTED
    assert call(rank=136) == nv.ERR_UNSUPPORTED
    assert call(rank=144) == nv.ERR_UNSUPPORTED
    assert call(K=(1 << 22) + 64) == nv.ERR_UNSUPPORTED
    assert call(down=A16 + 8) == nv.ERR_ALIGN
    assert call(up=A16 + 8) == nv.ERR_ALIGN
    assert call(K=96) == nv.ERR_UNSUPPORTED
    # the plain product's workspace is too small once L is added
    assert call(wsb=nv.workspace_bytes(nv.OP_GEMM_W4A4, 64, 64)) == nv.ERR_WORKSPACE
    assert call(M=0) == nv.OK


def test_svdq_and_channel_amax_validation():
    L = nv.lib()
    f = L.nvfp4_gemm_w4a4_svdq
    W = 1 << 30
    Q, R = nv.GEMM_QUANTIZE_ACT, nv.GEMM_REUSE_ACT

    def call(smooth=A16, rank=32, flags=Q, M=64, K=64):
        return f(A16, None, A16, A16, A4, smooth, A16, A16, rank, M, 64, K, A16, nv.BF16, flags, A16, W, None)

    assert call(smooth=None) == nv.ERR_NULL
    assert call(smooth=None, flags=R, M=0) == nv.OK            # reuse: smooth unused
    assert call(smooth=A16 + 4) == nv.ERR_ALIGN
    assert call(rank=0) == nv.ERR_SHAPE
    assert call(rank=24) == nv.ERR_UNSUPPORTED
    assert call(K=96) == nv.ERR_UNSUPPORTED
    assert call(M=0) == nv.OK
    c = L.nvfp4_channel_amax
    assert c(None, nv.BF16, 4, 64, A4, None) == nv.ERR_NULL
    assert c(A16, 3, 4, 64, A4, None) == nv.ERR_DTYPE
    assert c(A16, nv.BF16, 4, 24, A4, None) == nv.ERR_SHAPE
    assert c(A16 + 4, nv.BF16, 4, 64, A4, None) == nv.ERR_ALIGN
    assert c(A16, nv.BF16, 0, 64, A4, None) == nv.OK


def test_calibration_validation():
    L = nv.lib()
    W = nv.workspace_bytes(nv.OP_ACT_CALIBRATE, 64, 64)
    assert W > 0 and W % 256 == 0
    am = L.nvfp4_act_amax
    assert am(None, nv.BF16, 4, 64, A4, A16, W, None) == nv.ERR_NULL
    assert am(A16, nv.BF16, 4, 64, None, A16, W, None) == nv.ERR_NULL
    assert am(A16, 7, 4, 64, A4, A16, W, None) == nv.ERR_DTYPE
    assert am(A16, nv.BF16, 4, 40, A4, A16, W, None) == nv.ERR_SHAPE
    assert am(A16, nv.BF16, -1, 64, A4, A16, W, None) == nv.ERR_SHAPE
    assert am(A16 + 8, nv.BF16, 4, 64, A4, A16, W, None) == nv.ERR_ALIGN
    assert am(A16, nv.BF16, 4, 64, A4, A16, 0, None) == nv.ERR_WORKSPACE
    assert am(A16, nv.BF16, 0, 64, A4, A16, W, None) == nv.OK           # empty: no launch
    sw = L.nvfp4_act_scale_sweep
    assert sw(None, 4, 64, A4, A16, A4, A16, W, None) == nv.ERR_NULL
    assert sw(A16, 4, 64, A4, None, A4, A16, W, None) == nv.ERR_NULL
    assert sw(A16, 4, 64, A4, A16, None, A16, W, None) == nv.ERR_NULL
    assert sw(A16, 4, 24, A4, A16, A4, A16, W, None) == nv.ERR_SHAPE
    assert sw(A16, 4, 64, A4, A4, A4, A16, W, None) == nv.ERR_ALIGN     # errors must be 8-byte aligned
    assert sw(A16, 4, 64, A4, A16, A4, A16 + 16, W, None) == nv.ERR_ALIGN
    assert sw(A16, 4, 64, A4, A16, A4, A16, 8, None) == nv.ERR_WORKSPACE


def test_python_layer_rejects_mismatched_packed_shapes():
    import torch
    codes = torch.zeros((8, 32), dtype=torch.uint8)
    scales = torch.zeros((8, 4), dtype=torch.uint8)
    with pytest.raises(ValueError):
        nv._check_weight(codes, scales, 128)          # codes halved twice, as a BF16-read-as-FP4 mistake
    assert nv._check_weight(codes, scales, 64) == 8


def test_gemm_noalloc_validation():
    """The allocation-free W4A4 entry point checks its arguments like the
    workspace one, and refuses calls larger than its fixed scratch before
    any HIP call (the scratch is never looked up on these paths)."""
    f = nv.lib().nvfp4_gemm_w4a4_noalloc

    def call(a=A16, ag=None, wc=A16, ws=A4, wg=A4, M=64, N=64, K=64, y=A16, ydt=nv.BF16, flags=0):
        return f(a, ag, wc, ws, wg, M, N, K, y, ydt, flags, None)

    assert call(a=None) == nv.ERR_NULL
    assert call(a=None, flags=nv.GEMM_REUSE_ACT, M=0) == nv.OK     # reuse: a unused
    assert call(wc=None) == nv.ERR_NULL
    assert call(y=None) == nv.ERR_NULL
    assert call(flags=2) == nv.ERR_FLAGS
    assert call(ydt=5) == nv.ERR_DTYPE
    assert call(M=-1) == nv.ERR_SHAPE
    assert call(K=24) == nv.ERR_SHAPE
    assert call(K=96) == nv.ERR_UNSUPPORTED
    assert call(a=A16 + 4) == nv.ERR_ALIGN
    assert call(M=0) == nv.OK and call(N=0) == nv.OK
    # the largest activation that fits: workspace bytes <= NVFP4_NOALLOC_SCRATCH_BYTES
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4, 4096, 4096) <= nv.NOALLOC_SCRATCH_BYTES
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4, 4096, 12288) > nv.NOALLOC_SCRATCH_BYTES
    assert call(M=4096, K=12288) == nv.ERR_SCRATCH
    assert call(M=1 << 20, K=4096) == nv.ERR_SCRATCH
    assert nv.status_string(nv.ERR_SCRATCH).startswith("the call needs more than")
    m = re.search(r"#define NVFP4_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) \* 1024 \* 1024\)", open(HEADER).read())
    assert m and int(m.group(1)) * 1024 * 1024 == nv.NOALLOC_SCRATCH_BYTES


def test_gemm_group_validation():
    """Every product of a group is checked as nvfp4_gemm_w4a4 checks its
    arguments, before anything is launched; empty products need no launch."""
    f = nv.lib().nvfp4_gemm_w4a4_group
    W = nv.workspace_bytes(nv.OP_GEMM_W4A4, 64, 64)

    def prod(a=A16, ag=None, wc=A16, ws=A4, wg=A4, M=64, N=64, K=64, y=A16, flags=0, work=A16 * 16, wsb=W):
        return nv.GemmProduct(a, ag, wc, ws, wg, M, N, K, y, flags, work, wsb)

    def call(*ps, n=None, dt=nv.BF16):
        arr = (nv.GemmProduct * max(1, len(ps)))(*ps)
        return f(arr, len(ps) if n is None else n, dt, None)

    assert f(None, 0, nv.BF16, None) == nv.OK
    assert f(None, 1, nv.BF16, None) == nv.ERR_NULL
    assert call(prod(), n=-1) == nv.ERR_SHAPE
    assert call(prod(), dt=3) == nv.ERR_DTYPE
    assert call(prod(), prod(a=None)) == nv.ERR_NULL
    assert call(prod(a=None, flags=nv.GEMM_REUSE_ACT, M=0)) == nv.OK      # reuse: a unused
    assert call(prod(flags=4)) == nv.ERR_FLAGS
    assert call(prod(K=24)) == nv.ERR_SHAPE
    assert call(prod(K=96)) == nv.ERR_UNSUPPORTED
    assert call(prod(y=A16 + 4)) == nv.ERR_ALIGN
    assert call(prod(work=A16 * 16 + 16)) == nv.ERR_ALIGN
    assert call(prod(wsb=W - 1)) == nv.ERR_WORKSPACE
    assert call(prod(work=None)) == nv.ERR_NULL
    assert call(prod(M=0), prod(N=0)) == nv.OK


def test_empty_products_accept_null_pointers():
    """A product or dequantization with an empty output reads no pointer, so
    NULL ones are accepted (torch's zero-element tensors have NULL data
    pointers); sizes, dtypes and flags are still checked."""
    L = nv.lib()
    R = nv.GEMM_REUSE_ACT
    assert L.nvfp4_gemv_w4a16(None, None, None, None, 0, 64, 64, None, nv.BF16, None, 0, None) == nv.OK
    assert L.nvfp4_gemv_w4a16(None, None, None, None, 4, 0, 64, None, nv.BF16, None, 0, None) == nv.OK
    assert L.nvfp4_gemv_w4a16(None, None, None, None, 0, 64, 40, None, nv.BF16, None, 0, None) == nv.ERR_SHAPE
    assert L.nvfp4_gemv_w4a16(None, None, None, None, 0, 64, 64, None, 7, None, 0, None) == nv.ERR_DTYPE
    assert L.nvfp4_gemm_w4a4(None, None, None, None, None, 0, 64, 64, None, nv.BF16, 0, None, 0, None) == nv.OK
    assert L.nvfp4_gemm_w4a4(None, None, None, None, None, 64, 0, 64, None, nv.F32, R, None, 0, None) == nv.OK
    assert L.nvfp4_gemm_w4a4(None, None, None, None, None, 0, 64, 64, None, nv.BF16, 4, None, 0, None) == nv.ERR_FLAGS
    assert L.nvfp4_gemm_w4a4(None, None, None, None, None, 0, 64, 96, None, nv.BF16, 0, None, 0, None) == \
        nv.ERR_UNSUPPORTED
    assert L.nvfp4_gemm_w4a4_noalloc(None, None, None, None, None, 0, 64, 64, None, nv.BF16, 0, None) == nv.OK
    assert L.nvfp4_gemm_w4a4_lora(None, None, None, None, None, None, None, 32, 0, 64, 64, None, nv.BF16, 0, None,
                                  0, None) == nv.OK
    assert L.nvfp4_dequant(None, None, None, 0, 64, None, nv.BF16, None) == nv.OK
    assert L.nvfp4_dequant(None, None, None, 4, 0, None, nv.F32, None) == nv.OK
    assert L.nvfp4_dequant(None, None, None, 4, 64, None, nv.F32, None) == nv.ERR_NULL
    prods = (nv.GemmProduct * 2)(nv.GemmProduct(None, None, None, None, None, 0, 64, 64, None, 0, None, 0),
                                 nv.GemmProduct(None, None, None, None, None, 64, 0, 64, None, R, None, 0))
    assert L.nvfp4_gemm_w4a4_group(prods, 2, nv.BF16, None) == nv.OK
    # quantizers: an empty tensor needs no element pointers; a computed s_g is still written
    G = nv.GLOBAL_GIVEN
    assert L.nvfp4_quantize_absmax(None, nv.F32, 0, 64, None, None, None, G, None, 0, None) == nv.OK
    assert L.nvfp4_quantize_mse(None, nv.BF16, 8, 0, None, None, None, G, None, 0, None) == nv.OK
    assert L.nvfp4_quantize_4o6(None, nv.F32, 0, 64, None, None, None, 0, None, 0, None) == nv.ERR_NULL
    assert L.nvfp4_quantize_absmax(None, nv.F32, 0, 64, None, None, None, 0, None, 0, None) == nv.ERR_NULL
    assert L.nvfp4_quantize_absmax(None, nv.F32, 4, 64, None, None, A4, G, None, 0, None) == nv.ERR_NULL


def test_gemm_output_tile_limit():
    """At most 2^27 output tiles of 128 x 128 (grid and tile indices stay
    within 32 bits), checked before anything is launched, also per product of
    a group."""
    L = nv.lib()
    W = 1 << 40
    big = 1 << 30
    assert L.nvfp4_gemm_w4a4(A16, None, A16, A16, A4, big, big, 64, A16, nv.BF16, 0, A16, W, None) == \
        nv.ERR_UNSUPPORTED
    assert L.nvfp4_gemm_w4a4(A16, None, A16, A16, A4, 1 << 21, (1 << 20) + 128, 64, A16, nv.BF16, 0, A16, W, None) == \
        nv.ERR_UNSUPPORTED
    prods = (nv.GemmProduct * 1)(nv.GemmProduct(A16, None, A16, A16, A4, big, big, 64, A16, 0, A16, W))
    assert L.nvfp4_gemm_w4a4_group(prods, 1, nv.BF16, None) == nv.ERR_UNSUPPORTED

