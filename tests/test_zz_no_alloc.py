"""The allocation-free W4A4 entry point (nvfp4_gemm_w4a4_noalloc, fixed
per-GPU scratch) against the workspace entry point (nvfp4_gemm_w4a4), both
called through the C ABI: outputs bit-identical and within the oracle's tau,
on consecutive calls of decreasing size (the scratch keeps the previous
call's contents), a split-K product whose partial sums live in the scratch,
activation reuse from the previous call, and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from dit_quantization_amd import inputs
from dit_quantization_amd import nvfp4 as nv
from tests.gpu_helpers import DEV, assert_bracket_bf16, assert_within_tau, dev_bf16, host

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _weight(N, K, seed):
    oc, os_, og = oracle.quantize(inputs.student_t_f32((N, K), seed))
    return (oc, os_, og), (torch.from_numpy(oc).to(DEV), torch.from_numpy(os_).to(DEV),
                           torch.tensor([og], dtype=torch.float32, device=DEV))


def _noalloc(a, w, M, N, K, y, flags=0, ag=None):
    c, s, g = w
    return nv.lib().nvfp4_gemm_w4a4_noalloc(_p(a), _p(ag), _p(c), _p(s), _p(g), M, N, K, _p(y),
                                            nv.F32 if y.dtype == torch.float32 else nv.BF16, flags, _stream())


def _with_ws(a, w, M, N, K, y, ws, flags=0, ag=None):
    c, s, g = w
    return nv.lib().nvfp4_gemm_w4a4(_p(a), _p(ag), _p(c), _p(s), _p(g), M, N, K, _p(y),
                                    nv.F32 if y.dtype == torch.float32 else nv.BF16, flags, _p(ws), ws.numel(),
                                    _stream())


def _activation(M, K, seed):
    a = inputs.normal_f32((M, K), seed)
    a, _ = inputs.with_outlier_columns(a, max(1, K // 100), seed + 1)
    return inputs.to_bf16_bits(a)


def _compare(M, N, K, seed, ydt):
    print(f"[case] noalloc M={M} N={N} K={K} {ydt}", flush=True)
    ab = _activation(M, K, seed)
    (oc, os_, og), w = _weight(N, K, seed + 2)
    a = dev_bf16(ab)
    y0 = torch.full((M, N), 3.0, dtype=ydt, device=DEV)
    y1 = torch.full((M, N), 5.0, dtype=ydt, device=DEV)
    ws = torch.empty(nv.gemm_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    assert _noalloc(a, w, M, N, K, y0) == nv.OK
    assert _with_ws(a, w, M, N, K, y1, ws) == nv.OK
    torch.cuda.synchronize()
    assert np.array_equal(host(y0), host(y1))
    ac, as_, asg = oracle.quantize(inputs.bf16_bits_to_f32(ab))
    g = inputs.rng(seed + 5)
    pm, pn = g.integers(0, M, 400).astype(np.int64), g.integers(0, N, 400).astype(np.int64)
    ystar, tau = oracle.dot_w4a4(ac, as_, asg, oc, os_, og, K, pairs=(pm, pn), M=M, N=N)
    if ydt == torch.float32:
        assert_within_tau(host(y0)[pm, pn], ystar, tau, "noalloc fp32")
    else:
        assert_bracket_bf16(host(y0)[pm, pn], ystar, tau, "noalloc bf16")


def test_noalloc_matches_workspace_entry_point_on_shrinking_calls():
    # 4096 x 4096 fills half of the 64 MiB scratch; the next calls are smaller
    # and read a scratch that still holds the previous call's data
    _compare(4096, 1024, 4096, 101, torch.float32)
    _compare(300, 520, 1024, 102, torch.float32)
    _compare(70, 130, 192, 103, torch.bfloat16)


def test_noalloc_split_k_and_activation_reuse():
    """512 x 3072 x 12288 (the DiT text-stream MLP-down product) splits K into
    4 ranges whose partial sums sit in the scratch; a second weight then
    reuses the activation the first call quantized."""
    M, N, K = 512, 3072, 12288
    print(f"[case] noalloc split-K M={M} N={N} K={K}", flush=True)
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4, M, K) + 4 * M * N * 4 <= nv.NOALLOC_SCRATCH_BYTES
    ab = _activation(M, K, 104)
    _, w1 = _weight(N, K, 105)
    _, w2 = _weight(N, K, 106)
    a = dev_bf16(ab)
    ws = torch.empty(nv.gemm_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    outs = [torch.empty((M, N), dtype=torch.float32, device=DEV) for _ in range(4)]
    assert _noalloc(a, w1, M, N, K, outs[0]) == nv.OK
    assert _noalloc(None, w2, M, N, K, outs[1], flags=nv.GEMM_REUSE_ACT) == nv.OK
    assert _with_ws(a, w1, M, N, K, outs[2], ws) == nv.OK
    assert _with_ws(None, w2, M, N, K, outs[3], ws, flags=nv.GEMM_REUSE_ACT) == nv.OK
    torch.cuda.synchronize()
    assert np.array_equal(host(outs[0]), host(outs[2]))
    assert np.array_equal(host(outs[1]), host(outs[3]))


def test_noalloc_refuses_calls_beyond_its_scratch():
    M, N, K = 4096, 256, 12288          # 2 M K = 96 MiB of quantized activation
    a = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    (_, _, _), w = _weight(N, K, 107)
    y = torch.full((M, N), 9.0, dtype=torch.float32, device=DEV)
    assert _noalloc(a, w, M, N, K, y) == nv.ERR_SCRATCH
    torch.cuda.synchronize()
    assert np.all(host(y) == 9.0)
