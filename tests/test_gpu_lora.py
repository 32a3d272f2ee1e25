"""Parity of the fused low-rank (LoRA) W4A4 product with the oracle.

"NVFP4 en difusion ...", section 3: y = W_4bit x + B (A x) with the low-rank
term in 16 bits.  The tolerance adds the oracle's low-rank bound (bf16
rounding of L = x A^T, fp32 accumulation of both sums) to the W4A4 bound:
fp32 outputs within tau of y*, bf16 outputs inside [bf16(y* - tau),
bf16(y* + tau)].  L in the workspace is checked against the oracle's L*
(the low-rank term with B = I) within its own bound.
"""
import numpy as np
import pytest
import torch

import oracle
from dit_quantization_amd import inputs
from dit_quantization_amd import nvfp4 as nv
from tests.gpu_helpers import DEV, assert_bracket_bf16, assert_within_tau, dev_bf16, host

pytestmark = pytest.mark.gpu


def _quant_weight(w, method=oracle.MSE):
    """The oracle's NVFP4 encoding of w: (device tensors, host arrays)."""
    c, s, g = oracle.quantize(w, method)
    return (torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV),
            torch.tensor([g], dtype=torch.float32, device=DEV)), (c, s, g)


def _check_lora(ab, w, down_b, up_b, pairs=None, a_global=None, what="", method=oracle.MSE):
    M, K = ab.shape
    N, r = up_b.shape
    print(f"[case] gemm+lora {what} M={M} N={N} K={K} r={r}", flush=True)
    (c, s, g), (oc, os_, og) = _quant_weight(w, method)
    ws = torch.empty(nv.workspace_bytes(nv.OP_GEMM_W4A4_LORA, M, K), dtype=torch.uint8, device=DEV)
    a_dev, down, up = dev_bf16(ab), dev_bf16(down_b), dev_bf16(up_b)
    ag = None if a_global is None else torch.tensor([a_global], dtype=torch.float32, device=DEV)
    y32 = nv.gemm_w4a4(a_dev, c, s, g, a_global=ag, out_dtype=torch.float32, workspace=ws, lora=(down, up))
    torch.cuda.synchronize()
    a32 = inputs.bf16_bits_to_f32(ab)
    d32, u32 = inputs.bf16_bits_to_f32(down_b), inputs.bf16_bits_to_f32(up_b)
    wsh = host(ws)
    # quantized activation, as in the plain product
    ac, as_, asg = oracle.quantize(a32, oracle.ABSMAX, sg=a_global)
    assert wsh[:4].view(np.float32)[0] == np.float32(asg)
    ahat = wsh[256:256 + 2 * M * K].view(np.float16).reshape(M, K).astype(np.float32)
    assert np.array_equal(ahat, oracle.dequant(ac, as_, 1.0, M, K))
    # L = bf16(x A^T): within the oracle's bound for the low-rank term with B = I
    off = nv.gemm_lora_l_offset(M, K)
    L = wsh[off:off + 2 * M * r].view(np.uint16).reshape(M, r)
    lstar, ltau = oracle.lora_term(a32, d32, np.eye(r, dtype=np.float32))
    assert_within_tau(inputs.bf16_bits_to_f32(L).reshape(-1), lstar, ltau, what + " L")
    # products
    if pairs is None:
        ystar, tau = oracle.dot_w4a4(ac, as_, asg, oc, os_, og, K)
        lst, lt = oracle.lora_term(a32, d32, u32)
        sel = slice(None)
    else:
        ystar, tau = oracle.dot_w4a4(ac, as_, asg, oc, os_, og, K, pairs=pairs, M=M, N=N)
        lst, lt = oracle.lora_term(a32, d32, u32, pairs=pairs)
        sel = (pairs[0], pairs[1])
    ystar, tau = ystar + lst, tau + lt
    # the low-rank term must stand well above the tolerance, or the check proves nothing
    assert np.median(np.abs(lst)) > 5 * np.median(tau)
    assert_within_tau(host(y32)[sel].reshape(-1), ystar, tau, what + " fp32")
    yb = nv.gemm_w4a4(a_dev, c, s, g, a_global=ag, workspace=ws, lora=(down, up))
    assert_bracket_bf16(host(yb)[sel].reshape(-1), ystar, tau, what + " bf16")
    # reuse of the quantized activation and L from the workspace
    yr = nv.gemm_w4a4(a_dev, c, s, g, workspace=ws, reuse_act=True, lora=(down, up))
    assert np.array_equal(host(yr), host(yb))
    # the plain product on the same workspace reads the same quantized activation
    yp = nv.gemm_w4a4(a_dev, c, s, g, out_dtype=torch.float32, workspace=ws, reuse_act=True)
    assert_within_tau(host(yp)[sel].reshape(-1), ystar - lst, tau - lt, what + " plain")


# The down projection splits K over workgroups when there are few 16-row
# tiles: one range (M = 1, 70, 16400), 4 (M = 300), 32 (M = 257), 8 (M = 33)
# and 3 uneven ranges of 5, 5, 4 chunks (M = 40, K = 448).
@pytest.mark.parametrize("mnkr", [(1, 64, 64, 16), (70, 130, 192, 32), (300, 520, 512, 128), (257, 300, 4096, 48),
                                  (33, 96, 1024, 80), (40, 200, 448, 16), (16400, 64, 64, 16)])
def test_lora_ragged_full_compare(mnkr):
    M, N, K, r = mnkr
    a = inputs.normal_f32((M, K), M + 5)
    a, _ = inputs.with_outlier_columns(a, max(1, K // 100), 7)
    w = inputs.student_t_f32((N, K), N + 6)
    down, up = inputs.lora_factors(r, K, N, 100 + r, up_std=0.1)
    _check_lora(inputs.to_bf16_bits(a), w, down, up, what=str(mnkr))


def test_lora_static_activation_scale():
    a = inputs.normal_f32((96, 256), 11)
    w = inputs.student_t_f32((128, 256), 12)
    down, up = inputs.lora_factors(64, 256, 128, 13)
    _check_lora(inputs.to_bf16_bits(a), w, down, up, a_global=0.01, what="static s_gA")


def _sample_pairs(M, N, n, seed):
    g = inputs.rng(seed)
    pm = np.concatenate([[0, M - 1, 0, M - 1], g.integers(0, M, n)])
    pn = np.concatenate([[0, 0, N - 1, N - 1], g.integers(0, N, n)])
    return pm.astype(np.int64), pn.astype(np.int64)


@pytest.mark.parametrize("stream", [0, 1])
def test_lora_dit_block_sampled(stream):
    """Flux-like double-stream block layers with a rank-32 branch on each."""
    acts = inputs.dit_activations()
    a, h = acts[stream], acts[2 + stream]
    for i, (name, w) in enumerate(inputs.dit_weights(stream)):
        act = h if name == "mlp_down" else a
        M, K = act.shape
        N = w.shape[0]
        down, up = inputs.lora_factors(32, K, N, 200 + 10 * stream + i)
        _check_lora(act, w, down, up, pairs=_sample_pairs(M, N, 600, 50 + i), what=f"dit stream{stream} {name}",
                    method=oracle.ABSMAX)


def test_lora_rank_zero_branch_equals_plain():
    """A zero up-projection leaves exactly the plain W4A4 product."""
    ab = inputs.to_bf16_bits(inputs.normal_f32((200, 512), 3))
    (c, s, g), _ = _quant_weight(inputs.student_t_f32((320, 512), 4))
    down, _ = inputs.lora_factors(32, 512, 320, 5)
    up = torch.zeros((320, 32), dtype=torch.bfloat16, device=DEV)
    a = dev_bf16(ab)
    for dt in (torch.float32, torch.bfloat16):
        y_l = nv.gemm_w4a4(a, c, s, g, out_dtype=dt, lora=(dev_bf16(down), up))
        y_p = nv.gemm_w4a4(a, c, s, g, out_dtype=dt)
        assert np.array_equal(host(y_l), host(y_p))
