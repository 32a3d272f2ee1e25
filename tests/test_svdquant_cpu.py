"""Host-side SVDQuant preparation (no GPU): the smoothing factors equal the
oracle's, and the low-rank split has the properties the construction
guarantees (exact reconstruction up to the residual's rounding, an exact
low-rank weight leaves only bf16 rounding behind, the Eckart-Young tail,
outlier migration, and a user LoRA appended in the smoothed coordinates)."""
import numpy as np
import torch

import oracle
from dit_quantization_amd import inputs, svdquant


def _bits_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_smoothing_matches_oracle():
    g = inputs.rng(61)
    a = np.concatenate([g.uniform(0, 80, 4000), [0, 3, 5e-30]]).astype(np.float32)
    w = np.concatenate([g.uniform(0, 0.3, 4000), [1, 0, 2e-30]]).astype(np.float32)
    lam, smooth = svdquant.smoothing(a, w)
    olam, omult = oracle.smooth_factors(a, w)
    assert np.array_equal(lam, olam) and np.array_equal(smooth, omult)


def test_factors_reconstruct_and_tail():
    g = inputs.rng(62)
    w = inputs.student_t_f32((96, 160), 63)
    act = np.abs(g.standard_normal(160)).astype(np.float32) + 0.1
    act[::17] *= 20                                     # outlier channels
    f = svdquant.factors(w, act, 16)
    lam = f["lam"]
    ws = (w.astype(np.float64) * lam).astype(np.float32).astype(np.float64)
    p = _bits_f64(f["up"]) @ _bits_f64(f["down"])
    r = f["residual"].astype(np.float64)
    # R = fp32(W' - P): W' - P - R is R's own rounding error
    assert np.all(np.abs(ws - p - r) <= np.abs(r) * 2.0 ** -24)
    # the residual's energy is the SVD tail plus the factors' bf16 rounding
    s = np.linalg.svd(ws, compute_uv=False)
    tail = np.sqrt((s[16:] ** 2).sum())
    assert np.linalg.norm(r) <= tail + 2.0 ** -7 * np.linalg.norm(ws)
    assert np.linalg.norm(r) >= tail * (1 - 1e-3)       # no rank-16 matrix gets below the tail


def test_exact_low_rank_weight_leaves_only_rounding():
    g = inputs.rng(64)
    w = (g.standard_normal((128, 32)) @ g.standard_normal((32, 96)) * 0.01).astype(np.float32)
    act = np.abs(w).max(axis=0)                         # lambda = 1 everywhere
    f = svdquant.factors(w, act, 32)
    assert np.all(f["lam"] == 1.0) and np.all(f["smooth"] == 1.0)
    assert np.linalg.norm(f["residual"]) <= 2.0 ** -7 * np.linalg.norm(w)


def test_smoothing_migrates_outliers():
    """With strength 1/2 the smoothed activation range and the scaled weight
    range of every channel meet at sqrt(a_k w_k)."""
    g = inputs.rng(65)
    x = g.standard_normal((64, 128)).astype(np.float32)
    x[:, ::13] *= 30
    w = inputs.student_t_f32((48, 128), 66)
    a_k = np.abs(x).max(axis=0)
    w_k = np.abs(w).max(axis=0)
    lam, smooth = svdquant.smoothing(a_k, w_k)
    xs = np.abs(x * smooth).max(axis=0)
    wsc = np.abs(w * lam).max(axis=0)
    meet = np.sqrt(a_k.astype(np.float64) * w_k)
    assert np.allclose(xs, meet, rtol=1e-6) and np.allclose(wsc, meet, rtol=1e-6)
    # the outlier channels stand out far less against the typical channel
    assert xs.max() / np.median(xs) < (a_k.max() / np.median(a_k)) / 3


def test_user_lora_rides_along():
    g = inputs.rng(67)
    w = inputs.student_t_f32((64, 96), 68)
    act = np.abs(g.standard_normal(96)).astype(np.float32) + 0.5
    A = g.standard_normal((16, 96)).astype(np.float32) * 0.1
    B = g.standard_normal((64, 16)).astype(np.float32) * 0.1
    f = svdquant.factors(w, act, 16, lora=(A, B))
    assert f["down"].shape == (32, 96) and f["up"].shape == (64, 32)
    want_down = (torch.from_numpy((A.astype(np.float64) * f["lam"]).astype(np.float32))
                 .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(f["down"][16:], want_down)
    assert np.array_equal(f["up"][:, 16:], torch.from_numpy(B).to(torch.bfloat16).view(torch.int16).numpy()
                          .view(np.uint16))
