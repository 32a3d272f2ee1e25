"""GPU parity of the W4A16 GEMV and the W4A4 GEMM against the fp64 oracle:
fp32 outputs within tau = 1e-5 * sum |a||w| of y*, bf16 outputs inside
[bf16(y* - tau), bf16(y* + tau)]; the activation quantization inside the
W4A4 call is checked bit-exactly through its documented workspace."""
import numpy as np
import pytest
import torch

import oracle
from dit_quantization_amd import inputs
from dit_quantization_amd import nvfp4 as nv
from tests.gpu_helpers import DEV, assert_bracket_bf16, assert_within_tau, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


def _quant_weight(w, method=oracle.ABSMAX):
    """The oracle's NVFP4 encoding of w, uploaded: the products' weight inputs
    come from the oracle, never from the GPU quantizer."""
    c, s, g = oracle.quantize(w, method)
    dev = (torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV),
           torch.tensor([g], dtype=torch.float32, device=DEV))
    _ORACLE_WEIGHTS[dev[0].data_ptr()] = (c, s, g)
    return dev


_ORACLE_WEIGHTS = {}   # device codes pointer -> the oracle's (codes, scales, s_g) it was uploaded from


def _oracle_weight(c):
    return _ORACLE_WEIGHTS[c.data_ptr()]


def test_tiny_config_gemv():
    w, xb = inputs.tiny()
    gc, gs, _ = nv.quantize_absmax(dev_f32(w))      # the GPU quantizer on the tiny config ...
    c, s, g = _quant_weight(w)
    oc, os_, og = _oracle_weight(c)
    assert np.array_equal(host(gc), oc) and np.array_equal(host(gs), os_)   # ... matches the oracle's encoding
    x = inputs.bf16_bits_to_f32(xb)
    ystar, tau = oracle.dot_w4a16(x, oc, os_, og)
    yb = host(nv.gemv_w4a16(dev_bf16(xb), c, s, g))
    assert_bracket_bf16(yb.reshape(-1), ystar, tau, "tiny bf16")
    y32 = host(nv.gemv_w4a16(dev_bf16(xb), c, s, g, out_dtype=torch.float32))
    assert_within_tau(y32.reshape(-1), ystar, tau, "tiny fp32")


@pytest.mark.parametrize("shape", [(64, 32), (100, 160), (300, 96), (1000, 1056), (33, 4096)])
@pytest.mark.parametrize("M", [1, 3, 4, 5, 8, 16])
def test_gemv_ragged(shape, M):
    N, K = shape
    print(f"[case] gemv N={N} K={K} M={M}", flush=True)
    w = inputs.student_t_f32((N, K), N + K)
    xb = inputs.gemv_x(K, M)
    c, s, g = _quant_weight(w, oracle.MSE)
    oc, os_, og = _oracle_weight(c)
    ystar, tau = oracle.dot_w4a16(inputs.bf16_bits_to_f32(xb), oc, os_, og)
    y32 = host(nv.gemv_w4a16(dev_bf16(xb), c, s, g, out_dtype=torch.float32))
    assert_within_tau(y32.reshape(-1), ystar, tau, "fp32")
    yb = host(nv.gemv_w4a16(dev_bf16(xb), c, s, g))
    assert_bracket_bf16(yb.reshape(-1), ystar, tau, "bf16")


@pytest.mark.parametrize("shape", [(37, 6144), (20, 12320), (9, 32768), (70, 16384)])
def test_gemv_m1_long_rows(shape):
    """M = 1 with every row-length class of the single-row kernel: K <= 8192
    (2 chunks a lane), <= 16384 (4 chunks, 2 K parts; 12320 leaves K parts
    with idle lanes) and <= 32768 (4 K parts); N not a multiple of the 8 rows
    a workgroup covers."""
    N, K = shape
    print(f"[case] gemv M=1 N={N} K={K}", flush=True)
    w = inputs.student_t_f32((N, K), N + 3 * K)
    xb = inputs.gemv_x(K, 1)
    c, s, g = _quant_weight(w, oracle.MSE)
    oc, os_, og = _oracle_weight(c)
    ystar, tau = oracle.dot_w4a16(inputs.bf16_bits_to_f32(xb), oc, os_, og)
    y32 = host(nv.gemv_w4a16(dev_bf16(xb), c, s, g, out_dtype=torch.float32))
    assert_within_tau(y32.reshape(-1), ystar, tau, "fp32")
    assert_bracket_bf16(host(nv.gemv_w4a16(dev_bf16(xb), c, s, g)).reshape(-1), ystar, tau, "bf16")


@pytest.mark.parametrize("shape", [(300, 8320), (1000, 16384), (64, 8192)])
@pytest.mark.parametrize("M", [5, 16])
def test_gemv_splitk(shape, M):
    """M > 4 on short weights with long rows splits K (3 uneven ranges of
    17, 17, 17, 14 super-chunks for K = 8320; 8 for K = 16384; 4 for 64 rows):
    the split and the unsplit product both meet tau, the split one repeats."""
    N, K = shape
    print(f"[case] gemv split-K N={N} K={K} M={M}", flush=True)
    assert nv.workspace_bytes(nv.OP_GEMV_W4A16, M, N) > 0
    w = inputs.student_t_f32((N, K), N + K + 1)
    xb = inputs.gemv_x(K, M)
    oc, os_, og = oracle.quantize(w, oracle.MSE if N * K <= 1 << 22 else oracle.ABSMAX)
    c, s, g = torch.from_numpy(oc).to(DEV), torch.from_numpy(os_).to(DEV), torch.tensor([og], device=DEV)
    ystar, tau = oracle.dot_w4a16(inputs.bf16_bits_to_f32(xb), oc, os_, og)
    xd = dev_bf16(xb)
    y_split = host(nv.gemv_w4a16(xd, c, s, g, out_dtype=torch.float32))
    y_plain = host(nv.gemv_w4a16(xd, c, s, g, out_dtype=torch.float32, split_k=False))
    assert_within_tau(y_split.reshape(-1), ystar, tau, "split fp32")
    assert_within_tau(y_plain.reshape(-1), ystar, tau, "plain fp32")
    assert_bracket_bf16(host(nv.gemv_w4a16(xd, c, s, g)).reshape(-1), ystar, tau, "split bf16")
    assert np.array_equal(host(nv.gemv_w4a16(xd, c, s, g, out_dtype=torch.float32)), y_split)


@pytest.mark.parametrize("which", [0, 1])
def test_gemv_decode_full_size(which):
    w = inputs.gemv_weights()[which]
    N, K = w.shape
    print(f"[case] gemv full N={N} K={K}", flush=True)
    c, s, g = nv.quantize_absmax(dev_f32(w))
    oc, os_, og = oracle.quantize(w)
    assert float(host(g)[0]) == og
    assert np.array_equal(host(s), os_) and np.array_equal(host(c), oc)   # full-size absmax parity (so c, s, g are the oracle's)
    xb = inputs.gemv_x(K, 16)
    x = inputs.bf16_bits_to_f32(xb)
    ystar, tau = oracle.dot_w4a16(x, oc, os_, og)
    ystar = ystar.reshape(16, N)
    tau = tau.reshape(16, N)
    for M in (1, 4, 16):
        xd = dev_bf16(xb[:M])
        yb = host(nv.gemv_w4a16(xd, c, s, g))
        assert_bracket_bf16(yb.reshape(-1), ystar[:M].reshape(-1), tau[:M].reshape(-1), f"M={M}")
        y32 = host(nv.gemv_w4a16(xd, c, s, g, out_dtype=torch.float32))
        assert_within_tau(y32.reshape(-1), ystar[:M].reshape(-1), tau[:M].reshape(-1), f"M={M} fp32")


def _check_gemm(ab, w_c, w_s, w_g, pairs=None, a_global=None, what=""):
    M, K = ab.shape
    N = w_c.shape[0]
    print(f"[case] gemm {what} M={M} N={N} K={K}", flush=True)
    ws = torch.empty(nv.workspace_bytes(nv.OP_GEMM_W4A4, M, K), dtype=torch.uint8, device=DEV)
    a_dev = dev_bf16(ab)
    ag = None if a_global is None else torch.tensor([a_global], dtype=torch.float32, device=DEV)
    y32 = nv.gemm_w4a4(a_dev, w_c, w_s, w_g, a_global=ag, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    # activation quantization: s_gA and q_a * s_a (fp16) in the workspace
    a32 = inputs.bf16_bits_to_f32(ab)
    ac, as_, asg = oracle.quantize(a32, oracle.ABSMAX, sg=a_global)
    wsh = host(ws)
    assert wsh[:4].view(np.float32)[0] == np.float32(asg)
    ahat = wsh[256:256 + 2 * M * K].view(np.float16).reshape(M, K).astype(np.float32)
    want = oracle.dequant(ac, as_, 1.0, M, K)
    assert np.array_equal(ahat, want), np.argwhere(ahat != want)[:5]
    # products
    oc, os_, og = _oracle_weight(w_c)
    if pairs is None:
        ystar, tau = oracle.dot_w4a4(ac, as_, asg, oc, os_, og, K)
        sel = slice(None)
    else:
        ystar, tau = oracle.dot_w4a4(ac, as_, asg, oc, os_, og, K, pairs=pairs, M=M, N=N)
        sel = (pairs[0], pairs[1])
    assert_within_tau(host(y32)[sel].reshape(-1), ystar, tau, what + " fp32")
    yb = nv.gemm_w4a4(a_dev, w_c, w_s, w_g, a_global=ag, workspace=ws)
    assert_bracket_bf16(host(yb)[sel].reshape(-1), ystar, tau, what + " bf16")
    # the same product again from the activation already in the workspace
    yr = nv.gemm_w4a4(a_dev, w_c, w_s, w_g, workspace=ws, reuse_act=True)
    assert np.array_equal(host(yr), host(yb))


@pytest.mark.parametrize("mnk", [(1, 64, 64), (70, 130, 192), (300, 520, 512), (257, 300, 4096)])
def test_gemm_ragged_full_compare(mnk):
    M, N, K = mnk
    a = inputs.normal_f32((M, K), M + 1)
    a, _ = inputs.with_outlier_columns(a, max(1, K // 100), 3)
    ab = inputs.to_bf16_bits(a)
    w = inputs.student_t_f32((N, K), N + 2)
    c, s, g = _quant_weight(w, oracle.MSE)
    _check_gemm(ab, c, s, g, what=str(mnk))


def test_gemm_static_activation_scale():
    a = inputs.normal_f32((96, 256), 11)
    ab = inputs.to_bf16_bits(a)
    c, s, g = _quant_weight(inputs.student_t_f32((128, 256), 12))
    _check_gemm(ab, c, s, g, a_global=0.01, what="static s_gA")


def _sample_pairs(M, N, n, seed):
    g = inputs.rng(seed)
    pm = np.concatenate([[0, M - 1, 0, M - 1], g.integers(0, M, n)])
    pn = np.concatenate([[0, 0, N - 1, N - 1], g.integers(0, N, n)])
    return pm.astype(np.int64), pn.astype(np.int64)


def test_gemm_prefill_full_size_sampled():
    ab = inputs.prefill_activation()
    (_, w), = list(inputs.layerset(["gate"]))
    c, s, g = _quant_weight(w)
    _check_gemm(ab, c, s, g, pairs=_sample_pairs(4096, 14336, 3000, 1), what="prefill")


def test_gemm_dit_block_sampled():
    a_img, a_txt, h_img, h_txt = inputs.dit_activations()
    for stream, (a, h) in enumerate(((a_img, h_img), (a_txt, h_txt))):
        for name, w in inputs.dit_weights(stream):
            c, s, g = _quant_weight(w)
            act = h if name == "mlp_down" else a
            M, N = act.shape[0], w.shape[0]
            _check_gemm(act, c, s, g, pairs=_sample_pairs(M, N, 600, stream * 10 + len(name)),
                        what=f"dit stream{stream} {name}")


@pytest.mark.parametrize("mnk", [(70, 130, 1024), (300, 520, 4096), (33, 96, 4096), (100, 200, 1344),
                                 (512, 3072, 3072)])
def test_gemm_splitk_matches_oracle(mnk):
    """Short activations split K over workgroups when the workspace holds the
    partial sums; both the split and the unsplit product must meet tau, and
    the split one must repeat bit for bit."""
    M, N, K = mnk
    print(f"[case] gemm split-K M={M} N={N} K={K}", flush=True)
    assert nv.workspace_bytes(nv.OP_GEMM_W4A4_SPLITK, M, N) > 0
    a = inputs.normal_f32((M, K), M + 31)
    a, _ = inputs.with_outlier_columns(a, max(1, K // 100), 32)
    ab = inputs.to_bf16_bits(a)
    c, s, g = _quant_weight(inputs.student_t_f32((N, K), N + 33), oracle.MSE if N * K <= 1 << 22 else oracle.ABSMAX)
    a_dev = dev_bf16(ab)
    ws_split = torch.empty(nv.gemm_workspace_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    ws_plain = torch.empty(nv.gemm_workspace_bytes(M, N, K, split_k=False), dtype=torch.uint8, device=DEV)
    y_split = nv.gemm_w4a4(a_dev, c, s, g, out_dtype=torch.float32, workspace=ws_split)
    y_plain = nv.gemm_w4a4(a_dev, c, s, g, out_dtype=torch.float32, workspace=ws_plain)
    yb_split = nv.gemm_w4a4(a_dev, c, s, g, workspace=ws_split)
    torch.cuda.synchronize()
    ac, as_, asg = oracle.quantize(inputs.bf16_bits_to_f32(ab), oracle.ABSMAX)
    oc, os_, og = _oracle_weight(c)
    if M * N > 200000:
        pairs = _sample_pairs(M, N, 4000, 5)
        ystar, tau = oracle.dot_w4a4(ac, as_, asg, oc, os_, og, K, pairs=pairs, M=M, N=N)
        sel = (pairs[0], pairs[1])
    else:
        ystar, tau = oracle.dot_w4a4(ac, as_, asg, oc, os_, og, K)
        sel = slice(None)
    assert_within_tau(host(y_split)[sel].reshape(-1), ystar, tau, "split fp32")
    assert_within_tau(host(y_plain)[sel].reshape(-1), ystar, tau, "plain fp32")
    assert_bracket_bf16(host(yb_split)[sel].reshape(-1), ystar, tau, "split bf16")
    y_again = nv.gemm_w4a4(a_dev, c, s, g, out_dtype=torch.float32, workspace=ws_split)
    assert np.array_equal(host(y_again), host(y_split))


def test_gemm_and_gemv_deterministic():
    ab = inputs.to_bf16_bits(inputs.normal_f32((256, 512), 1))
    c, s, g = _quant_weight(inputs.student_t_f32((384, 512), 2))
    y1 = host(nv.gemm_w4a4(dev_bf16(ab), c, s, g))
    y2 = host(nv.gemm_w4a4(dev_bf16(ab), c, s, g))
    assert np.array_equal(y1, y2)
    v1 = host(nv.gemv_w4a16(dev_bf16(ab[:16]), c, s, g))
    v2 = host(nv.gemv_w4a16(dev_bf16(ab[:16]), c, s, g))
    assert np.array_equal(v1, v2)


@pytest.mark.parametrize("which", [0, 1])
def test_gemv_deterministic_decode_shapes(which):
    """Every GEMV kernel repeats bit for bit at full size (M = 1, 4, 16 on both
    decode shapes, fp32 out, ten calls each; rotating two weight copies so
    the calls read from HBM)."""
    w = inputs.gemv_weights()[which]
    N, K = w.shape
    c, s, g = _quant_weight(w)
    copies = [(c, s), (c.clone(), s.clone())]
    xb = dev_bf16(inputs.gemv_x(K, 16))
    for M in (1, 4, 16):
        print(f"[case] gemv repeat N={N} K={K} M={M}", flush=True)
        outs = [host(nv.gemv_w4a16(xb[:M].contiguous(), cc, ss, g, out_dtype=torch.float32))
                for i in range(10) for cc, ss in [copies[i % 2]]]
        for o in outs[1:]:
            assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("M", [1, 5])
def test_gemv_maximum_k(M):
    """K = 2^24, the largest the decode product accepts (N = 16 rows; M = 5 also
    splits K into 8 ranges)."""
    N, K = 16, 1 << 24
    print(f"[case] gemv max K N={N} K={K} M={M}", flush=True)
    w = inputs.normal_f32((N, K), 77, std=0.02)
    c, s, g = _quant_weight(w)
    del w
    oc, os_, og = _oracle_weight(c)
    xb = inputs.gemv_x(K, M)
    ystar, tau = oracle.dot_w4a16(inputs.bf16_bits_to_f32(xb), oc, os_, og)
    y32 = host(nv.gemv_w4a16(dev_bf16(xb), c, s, g, out_dtype=torch.float32))
    assert_within_tau(y32.reshape(-1), ystar, tau, "max K fp32")


def test_gemm_maximum_k():
    """K = 2^22, the largest the W4A4 product accepts (M = N = 16), split into
    8 K ranges and unsplit."""
    M, N, K = 16, 16, 1 << 22
    print(f"[case] gemm max K M={M} N={N} K={K}", flush=True)
    ab = inputs.to_bf16_bits(inputs.normal_f32((M, K), 78))
    c, s, g = _quant_weight(inputs.normal_f32((N, K), 79, std=0.02))
    oc, os_, og = _oracle_weight(c)
    ac, as_, asg = oracle.quantize(inputs.bf16_bits_to_f32(ab), oracle.ABSMAX)
    ystar, tau = oracle.dot_w4a4(ac, as_, asg, oc, os_, og, K)
    del ac, as_
    a_dev = dev_bf16(ab)
    for split in (True, False):
        ws = torch.empty(nv.gemm_workspace_bytes(M, N, K, split_k=split), dtype=torch.uint8, device=DEV)
        y32 = host(nv.gemm_w4a4(a_dev, c, s, g, out_dtype=torch.float32, workspace=ws))
        assert_within_tau(y32.reshape(-1), ystar, tau, f"max K split={split}")
