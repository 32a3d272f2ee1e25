"""Pins for the CPU oracle against what the pages and mathematics fix.

Every test here runs without a GPU.  The oracle is never compared with itself:
each check uses the pages' printed values (tests/golden/), a library routine
(torch's float8_e4m3fn / bfloat16 casts, numpy float64 matmul), an independent
exact-rational implementation (oracle/exact.py), closed forms or invariants.
"""
import math
import os
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle
from oracle import exact
from dit_quantization_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- formats

def test_e2m1_decode_matches_page_grid():
    for code, val in _read("e2m1_grid.txt"):
        got = oracle.e2m1_value(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code
    distinct = {abs(oracle.e2m1_value(c)) for c in range(16)}
    assert sorted(distinct) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_decode_matches_torch_all_bytes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        got = oracle.e4m3_value(b)
        if math.isnan(ref[b]):
            assert math.isnan(got), b
        else:
            assert got == ref[b], b
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_nearest_matches_torch_cast():
    g = inputs.rng(123)
    vals = list(g.uniform(0, 460, 4000)) + list(np.exp(g.uniform(-16, 6, 4000)))
    # every midpoint between adjacent E4M3 values, and its fp32 neighbours
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    for lo, hi in zip(e4[:-1], e4[1:]):
        m = np.float32((lo + hi) / 2)
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    vals = np.array(vals, dtype=np.float32)
    vals = vals[vals <= 448.0]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_nearest(float(v)) for v in vals])
    assert np.array_equal(got, ref)


def test_e4m3_nearest_saturates():
    for v in (448.0, 463.9, 464.0, 480.0, 1e6, 1e300):
        assert oracle.e4m3_nearest(v) == 0x7E


def test_e4m3_nearest_matches_exact_rounding():
    g = inputs.rng(7)
    for v in list(np.exp(g.uniform(-12, 7, 3000))) + [2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -11]:
        want = exact.round_format(F(float(v)), 3, -6, exact.E4M3_MAX)
        assert oracle.e4m3_value(oracle.e4m3_nearest(float(v))) == float(want), v


def test_e2m1_nearest_ties_and_neighbours_exact():
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 6.0, 7.0, 100.0, 0.0]
    xs = []
    for p in pts:
        xs += [p, -p, np.nextafter(p, 0), np.nextafter(p, 1e9), -np.nextafter(p, 0), -np.nextafter(p, 1e9)]
    xs += list(inputs.rng(5).uniform(-8, 8, 5000))
    for x in xs:
        want = exact.e2m1_code(exact.round_format(F(float(x)), 1, 0, exact.E2M1_MAX))
        assert oracle.e2m1_nearest(float(x)) == want, x
    # printed tie rule: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    for x, v in [(0.25, 0), (0.75, 1), (1.25, 1), (1.75, 2), (2.5, 2), (3.5, 4), (5.0, 4)]:
        assert oracle.e2m1_value(oracle.e2m1_nearest(x)) == v
        assert oracle.e2m1_value(oracle.e2m1_nearest(-x)) == -v
    assert oracle.e2m1_nearest(-0.1) == 0  # canonical +0


def test_bf16_rounding_helper_matches_torch():
    g = inputs.rng(9)
    v = np.concatenate([g.standard_normal(20000), g.standard_normal(2000) * 1e-30, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8])])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_rne_from_f64(v32.astype(np.float64))
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- global scale

def test_global_scale_exact():
    g = inputs.rng(11)
    for amax in list(g.uniform(0, 10, 2000).astype(np.float32)) + [np.float32(2688.0), np.float32(1e-38)]:
        want = exact.global_scale(F(float(amax)))
        assert oracle.global_scale(float(amax)) == float(want), amax
    assert oracle.global_scale(0.0) == 1.0


# ---------------------------------------------------------------- quantizer

def _blocks_tiny(seed, n):
    g = inputs.rng(seed)
    out = []
    for i in range(n):
        kind = i % 4
        if kind == 0:
            b = g.standard_normal(16) * 0.02
        elif kind == 1:
            b = g.standard_t(5, 16) * 0.02
        elif kind == 2:
            b = g.standard_normal(16) * 0.02
            b[0] *= (1, 3, 6, 12, 30)[i % 5]      # outlier factors of the toy experiment
        else:
            b = np.exp(g.uniform(-30, 5, 16)) * g.choice([-1, 1], 16)
        out.append(b.astype(np.float32))
    return np.stack(out)


def test_quantize_absmax_matches_exact_rational():
    x = _blocks_tiny(1, 96).reshape(6, 256)
    codes, scales, sg = oracle.quantize(x, oracle.ABSMAX)
    assert sg == float(exact.global_scale(F(float(np.abs(x).max()))))
    for r in range(x.shape[0]):
        for j in range(x.shape[1] // 16):
            blk = [F(float(v)) for v in x[r, 16 * j:16 * j + 16]]
            sb = exact.absmax_scale(blk, F(sg))
            assert scales[r, j] == exact.E4M3_INDEX[sb]
            cs = exact.codes_for(blk, sb, F(sg))
            packed = [cs[2 * i] | (cs[2 * i + 1] << 4) for i in range(8)]
            assert list(codes[r, 8 * j:8 * j + 8]) == packed


def test_quantize_exact_ties_in_codes_and_scales():
    # s_g = 1 given; blocks built so that W / s_b hits every E2M1 midpoint, and
    # amax / 6 hits E4M3 midpoints exactly.
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    rows = []
    for c in (8, 20, 0x38, 60, 100, 125):
        sb = e4[c]
        mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
        row = [6 * sb] + [m * sb for m in mids] + [-m * sb for m in mids] + [0.0]
        rows.append(row)
    for lo, hi in zip(e4[1:-1:7], e4[2::7]):
        mid = (lo + hi) / 2
        rows.append([6 * mid] + [0.0] * 15)
    x = np.array(rows, dtype=np.float32)
    codes, scales, sg = oracle.quantize(x, oracle.ABSMAX, sg=1.0)
    for r in range(x.shape[0]):
        blk = [F(float(v)) for v in x[r]]
        sb = exact.absmax_scale(blk, F(1))
        assert scales[r, 0] == exact.E4M3_INDEX[sb]
        cs = exact.codes_for(blk, sb, F(1))
        assert list(codes[r]) == [cs[2 * i] | (cs[2 * i + 1] << 4) for i in range(8)]


def test_pack_example_golden():
    rows = {r[0]: r[1:] for r in _read("pack_example.txt")}
    x = np.array([float(v) for v in rows["input"]], dtype=np.float32).reshape(1, 32)
    codes, scales, _ = oracle.quantize(x, oracle.ABSMAX, sg=1.0)
    assert [f"{b:02X}" for b in codes[0]] == rows["codes"]
    assert [f"{b:02X}" for b in scales[0]] == rows["scales"]


def test_mse_matches_exact_bruteforce_and_beats_absmax():
    x = _blocks_tiny(2, 64)
    sg = F(oracle.global_scale(float(np.abs(x).max())))
    outside = 0
    for blk_np in x:
        blk = [F(float(v)) for v in blk_np]
        best, best_err, gbest, gbest_err = exact.mse_search(blk, sg)
        code = oracle.mse_scale_code(blk_np, float(sg))
        chosen = exact.E4M3[code]
        chosen_err = exact.block_error(blk, chosen, sg)
        # oracle's fp64 choice is the exact windowed optimum (or an exact tie of it)
        assert chosen_err == best_err or abs(chosen_err - best_err) <= best_err * F(1, 10 ** 12), (code, best)
        # MSE never worse than absmax, exactly
        abs_err = exact.block_error(blk, exact.absmax_scale(blk, sg), sg)
        assert chosen_err <= abs_err
        outside += gbest != best
    # the unrestricted optimum is reported, not gated
    print(f"blocks whose unrestricted optimum lies outside [a/2, 2a]: {outside}/{len(x)}")


def test_four_over_six_matches_exact_and_never_worse_than_absmax():
    x = _blocks_tiny(5, 64)
    sg = F(oracle.global_scale(float(np.abs(x).max())))
    picked_four = 0
    for blk_np in x:
        blk = [F(float(v)) for v in blk_np]
        best, best_err = exact.four_over_six(blk, sg)
        code = oracle.four_over_six_scale_code(blk_np, float(sg))
        chosen = exact.E4M3[code]
        chosen_err = exact.block_error(blk, chosen, sg)
        # the oracle's fp64 choice is the exact choice, or an exact-or-rounding tie of it
        assert chosen == best or abs(chosen_err - best_err) <= best_err * F(1, 10 ** 12), (code, best)
        abs_scale = exact.absmax_scale(blk, sg)
        assert chosen_err <= exact.block_error(blk, abs_scale, sg)
        picked_four += chosen != abs_scale
    assert picked_four > 0          # the second candidate does win on some blocks


def test_four_over_six_worked_block():
    # s_g = 1, one 6.0 and fifteen 5.0.  Max -> 6 (scale 1.0, code 0x38): each
    # 5 sits on the 4|6 midpoint and rounds to the even code (4), error 1 each,
    # total 15.  Max -> 4 (scale 1.5, code 0x3C): 5 / 1.5 = 3.33 -> 3, i.e.
    # 4.5, error 0.25 each, total 3.75; the 6 maps to 4 exactly.  Four wins.
    blk = np.full(16, 5.0, dtype=np.float32)
    blk[0] = 6.0
    assert oracle.block_error(blk, 1.0, 0x38) == 15.0
    assert oracle.block_error(blk, 1.0, 0x3C) == 3.75
    assert oracle.four_over_six_scale_code(blk, 1.0) == 0x3C
    # sixteen 6.0: both candidates reconstruct exactly -> tie -> the smaller scale
    assert oracle.four_over_six_scale_code(np.full(16, 6.0, dtype=np.float32), 1.0) == 0x38
    # all-zero block: scale 0
    assert oracle.four_over_six_scale_code(np.zeros(16, dtype=np.float32), 1.0) == 0


def test_four_over_six_tensor_method_matches_block_function():
    x = _blocks_tiny(6, 32).reshape(8, 64)
    c, s, sg = oracle.quantize(x, oracle.FOUR_OVER_SIX)
    for r in range(8):
        for b in range(4):
            blk = x[r, 16 * b:16 * b + 16]
            assert s[r, b] == oracle.four_over_six_scale_code(blk, sg)


def test_mse_window_bounds_are_exact_e4m3_steps():
    # a block whose a = amax/(6 s_g) is itself an E4M3 value: the window holds
    # exactly 17 candidates (a/2 .. 2a inclusive) in the normal range.
    blk = np.zeros(16, dtype=np.float32)
    blk[0] = 6.0
    a = 1.0
    n = sum(1 for c in range(1, 127) if a / 2 <= oracle.e4m3_value(c) <= 2 * a)
    assert n == 17
    assert oracle.mse_scale_code(blk, 1.0) == 0x38  # exact representation wins (zero error)


def _random_f32_scales(seed, n):
    """fp32 tensor scales with full 24-bit significands over many binades."""
    g = inputs.rng(seed)
    sig = g.integers(2 ** 23, 2 ** 24, n)
    return [float(np.float32(np.ldexp(float(m), int(e)))) for m, e in zip(sig, g.integers(-40, -10, n))]


def test_mse_candidate_union_at_the_e4m3_cap():
    """Given s_g = 1 and max|W| = 6000, a = max|W| / (6 s_g) = 1000: the window
    [a/2, min(2a, 448)] = [500, 448] holds no E4M3 value, so the absmax scale
    (448, the saturated nearest value, byte 0x7E) is the only candidate
    ("Tu pipeline NVFP4 ...", section 2, box on MSE vs absmax: the searched
    scale is never worse than the absmax one, here because it is the absmax
    one).  Without the absmax scale in the candidate set the search would
    have no candidate at all."""
    g = inputs.rng(61)
    for i in range(24):
        blk = (g.standard_normal(16) * 1000).astype(np.float32)
        blk[i % 16] = np.float32(6000.0 if i % 2 == 0 else -6000.0)
        if i >= 16:
            blk *= np.float32(1 + i)          # a up to 25000: still only the capped absmax scale
        sg = F(1)
        code = oracle.mse_scale_code(blk, 1.0)
        assert code == 0x7E, (i, code)
        assert code == oracle.absmax_scale_code(blk, 1.0)
        fb = [F(float(v)) for v in blk]
        best, best_err, _, _ = exact.mse_search(fb, sg)
        assert best == exact.E4M3[code] == 448
        assert exact.block_error(fb, exact.E4M3[code], sg) <= exact.block_error(fb, exact.absmax_scale(fb, sg), sg)
    # the same cap reached under a general s_g: max|W| = 1500 * 6 * s_g
    for sg_f in _random_f32_scales(62, 8):
        blk = (g.standard_normal(16) * 200 * sg_f).astype(np.float32)
        blk[3] = np.float32(9000 * sg_f)
        code = oracle.mse_scale_code(blk, sg_f)
        fb = [F(float(v)) for v in blk]
        best, _, _, _ = exact.mse_search(fb, F(sg_f))
        assert code == 0x7E and best == 448, (sg_f, code)


def test_mse_candidate_union_below_the_smallest_subnormal_scale():
    """a = max|W| / (6 s_g) below 2^-10 (half the smallest positive E4M3 value
    2^-9): the absmax scale rounds to 0 and the window [a/2, 2a] holds no
    positive E4M3 value, so scale byte 0 (every code 0) is the only candidate
    and the MSE search must return it."""
    g = inputs.rng(63)
    e4_min = 2.0 ** -9
    for i, a_target in enumerate([2.0 ** -12, 2.0 ** -11, 0.9 * 2.0 ** -10, 0.999 * 2.0 ** -10, 1e-6, 2.0 ** -30]):
        blk = (g.uniform(-1, 1, 16) * 6 * a_target).astype(np.float32)
        blk[i] = np.float32(6 * a_target)
        a = float(np.abs(blk).max()) / 6.0
        assert 2 * a < e4_min                 # the window is empty
        code = oracle.mse_scale_code(blk, 1.0)
        assert code == 0 == oracle.absmax_scale_code(blk, 1.0), (a_target, code)
        fb = [F(float(v)) for v in blk]
        best, best_err, _, _ = exact.mse_search(fb, F(1))
        assert best == 0 and best_err == exact.block_error(fb, F(0), F(1))
    # and through the tensor entry point: scale bytes 0x00 and 0x7E, never 0xFF
    rows = np.zeros((2, 16), dtype=np.float32)
    rows[0, :] = np.float32(2.0 ** -13)
    rows[1, 0] = np.float32(6000.0)
    codes, scales, _ = oracle.quantize(rows, oracle.MSE, sg=1.0)
    assert list(scales[:, 0]) == [0x00, 0x7E]
    assert not codes[0].any()


def test_worked_example_levels():
    # s_b * s_g = 0.01 with s_g = 0.01 given and s_b = 1.0 (E4M3 0x38)
    levels = sorted({float(r[0]) for r in _read("worked_example_scale_0p01.txt")})
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8).reshape(1, 8)
    deq = oracle.dequant(packed, np.array([[0x38]], dtype=np.uint8), 0.01, 1, 16)[0]
    got = sorted({float(v) for v in deq})
    assert len(got) == len(levels) == 15
    for g_, l_ in zip(got, levels):
        assert abs(g_ - l_) <= 1e-7 * max(abs(l_), 1e-30)


def test_roundtrip_of_representable_values():
    g = inputs.rng(3)
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    rows = []
    for _ in range(40):
        c = int(g.integers(1, 127))
        q = g.choice(grid, 16) * g.choice([-1, 1], 16)
        q[int(g.integers(16))] = 6 * g.choice([-1, 1])
        rows.append(q * e4[c])
    x = np.array(rows, dtype=np.float32).reshape(-1, 16)
    assert np.all(x == np.array(rows))         # values representable in fp32
    codes, scales, _ = oracle.quantize(x, oracle.ABSMAX, sg=1.0)
    back = oracle.dequant(codes, scales, 1.0, x.shape[0], 16)
    assert np.array_equal(back, x)
    codes_m, scales_m, _ = oracle.quantize(x, oracle.MSE, sg=1.0)
    assert np.array_equal(oracle.dequant(codes_m, scales_m, 1.0, x.shape[0], 16), x)


def test_memory_accounting_4p5_bits():
    for params, bf16_gb, nv_gb, tol in _read("memory_accounting.txt"):
        n = int(float(params))
        rows, cols = 1, n  # the byte count depends only on the element count
        nbytes = rows * cols // 2 + rows * cols // 16
        assert abs(n * 2 / 1e9 - float(bf16_gb)) < 1e-9
        assert abs(nbytes / 1e9 - float(nv_gb)) <= float(tol)
        assert nbytes * 8 / n == 4.5
    # the oracle's output layout: [R, C/2] codes + [R, C/16] scales
    codes, scales, _ = oracle.quantize(np.ones((48, 160), np.float32))
    total = codes.nbytes + scales.nbytes
    assert total == 48 * 160 * (0.5 + 0.0625)
    assert abs(scales.nbytes / total - 1 / 9) < 1e-12        # "11 %"


# ---------------------------------------------------------------- products

def test_dot_w4a16_one_hot_gives_dequant_row():
    w = inputs.normal_f32((8, 64), 4, 0.02)
    codes, scales, sg = oracle.quantize(w)
    wh = oracle.dequant(codes, scales, sg, 8, 64).astype(np.float64)
    x = np.eye(64, dtype=np.float32)[:5]
    y, tau = oracle.dot_w4a16(x, codes, scales, sg)
    y = y.reshape(5, 8)
    # exact products: the one-hot picks W^[n, k] exactly (fp32-rounded dequant differs by < 1 ulp)
    assert np.allclose(y, wh[:, :5].T, rtol=2 ** -23, atol=0)


def test_dot_products_small_integer_exact_and_numpy_crosscheck():
    g = inputs.rng(6)
    K = 64
    # operands whose NVFP4 encoding is exact (s_g = 1, scale 1.0 per block)
    qa = g.choice([0, 0.5, 1, 1.5, 2, 3, 4, 6], (3, K)) * g.choice([-1, 1], (3, K))
    qw = g.choice([0, 0.5, 1, 1.5, 2, 3, 4, 6], (5, K)) * g.choice([-1, 1], (5, K))
    qa[:, ::16] = 6
    qw[:, ::16] = -6
    ac, as_, _ = oracle.quantize(qa.astype(np.float32), sg=1.0)
    wc, ws, _ = oracle.quantize(qw.astype(np.float32), sg=1.0)
    y, tau = oracle.dot_w4a4(ac, as_, 1.0, wc, ws, 1.0, K)
    assert np.array_equal(y.reshape(3, 5), qa @ qw.T)          # exact small-integer result
    y16, _ = oracle.dot_w4a16(qa.astype(np.float32), wc, ws, 1.0)
    assert np.array_equal(y16.reshape(3, 5), qa @ qw.T)
    # random operands: numpy float64 matmul of the dequantized operands
    a = inputs.normal_f32((7, 256), 8)
    w = inputs.student_t_f32((9, 256), 9)
    ac, as_, sga = oracle.quantize(a)
    wc, ws, sgw = oracle.quantize(w, oracle.MSE)
    ah = oracle.dequant(ac, as_, sga, 7, 256).astype(np.float64)
    whh = oracle.dequant(wc, ws, sgw, 9, 256).astype(np.float64)
    y, tau = oracle.dot_w4a4(ac, as_, sga, wc, ws, sgw, 256)
    ref = ah @ whh.T
    assert np.allclose(y.reshape(7, 9), ref, rtol=0, atol=1e-6 * (np.abs(ah) @ np.abs(whh).T).max())
    assert np.all(tau > 0)


def _exact_dequant(codes, scales, sg, rows, cols):
    """Exact rationals q * s_b * s_g, decoded with the exact checker's own
    E2M1 and E4M3 tables (independent of the C oracle)."""
    out = []
    for r in range(rows):
        row = []
        for k in range(cols):
            byte = int(codes[r, k // 2])
            c = (byte >> 4) if k & 1 else (byte & 15)
            mag = exact.E2M1_MAG[c & 7] * exact.E4M3[int(scales[r, k // 16])] * F(sg)
            row.append(-mag if c & 8 else mag)
        out.append(row)
    return out


def test_dequant_is_one_rounding_of_the_exact_product():
    """W^ = q s_b s_g ("Tu pipeline NVFP4 ...", section 2, the hierarchical
    reconstruction) rounded once to fp32: every code x every finite positive
    scale byte x 128 fp32 tensor scales with full significands.  Rounding
    s_b s_g to fp32 before the multiply by q (a double rounding) fails here."""
    codes = np.tile(np.array([c | ((c + 1) << 4) for c in range(0, 16, 2)], dtype=np.uint8), (127, 1))
    scales = np.arange(127, dtype=np.uint8).reshape(127, 1)
    sgs = _random_f32_scales(64, 120) + [1.0, 0.01, 3.0 / 7.0, 1e-30, 2.0 ** 100,
                                         float(np.nextafter(np.float32(1), np.float32(2)))]
    for sg in (float(np.float32(v)) for v in sgs):
        got = oracle.dequant(codes, scales, sg, 127, 16)
        want = _exact_dequant(codes, scales, sg, 127, 16)
        for r in range(127):
            for k in range(16):
                assert got[r, k] == float(exact.fp32(want[r][k])), (sg, r, k)


def test_one_hot_products_equal_the_exact_dequantized_weight():
    """A one-hot activation picks one weight element, whose exact value
    q s_b s_g has at most 30 significant bits, so the fp64 product sum must
    equal it exactly (rtol 0), and its tolerance must be 1e-5 |W^| rounded
    once (the product tolerance at one nonzero term)."""
    w = inputs.student_t_f32((6, 64), 65)
    for sg in _random_f32_scales(66, 6) + [None]:
        codes, scales, sgw = oracle.quantize(w, oracle.MSE, sg=sg)
        want = _exact_dequant(codes, scales, sgw, 6, 64)
        x = np.zeros((64, 64), dtype=np.float32)
        x[np.arange(64), np.arange(64)] = 1.0
        y, tau = oracle.dot_w4a16(x, codes, scales, sgw)
        y, tau = y.reshape(64, 6), tau.reshape(64, 6)
        for k in range(64):
            for n in range(6):
                assert y[k, n] == float(want[n][k]), (sg, k, n)
                assert tau[k, n] == 1e-5 * abs(float(want[n][k])), (sg, k, n)
        # W4A4: a one-hot activation block [6, 0, ...] quantizes exactly at
        # s_gA = 1 (scale 1.0, code 6), so y* = 6 W^ exactly
        a = np.zeros((16, 64), dtype=np.float32)
        a[np.arange(16), 4 * np.arange(16)] = 6.0
        ac, as_, _ = oracle.quantize(a, sg=1.0)
        y4, t4 = oracle.dot_w4a4(ac, as_, 1.0, codes, scales, sgw, 64)
        y4, t4 = y4.reshape(16, 6), t4.reshape(16, 6)
        for m in range(16):
            for n in range(6):
                assert y4[m, n] == float(6 * want[n][4 * m])
                assert t4[m, n] == 1e-5 * abs(float(6 * want[n][4 * m]))


def test_product_tolerance_matches_exact_rational():
    """tau = 1e-5 sum_k |a^_k| |w^_k| over the fully dequantized operands, and
    y* = sum_k a^_k w^_k, recomputed in exact rationals from the exact
    checker's decode (random operands, general tensor scales, W4A16 and
    W4A4).  The fp64 sums may differ from the exact ones only by their
    rounding (far below 1e-12 relative)."""
    K = 96
    g = inputs.rng(67)
    w = (g.standard_t(5, (5, K)) * 0.02).astype(np.float32)
    a = (g.standard_normal((4, K)) * np.where(g.uniform(size=K) < 0.1, 20.0, 1.0)).astype(np.float32)
    xb = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(a))
    wc, ws, sgw = oracle.quantize(w, oracle.MSE)
    ac, as_, sga = oracle.quantize(a)
    W = _exact_dequant(wc, ws, sgw, 5, K)
    A = _exact_dequant(ac, as_, sga, 4, K)
    tol = F(1, 10 ** 12)
    y16, t16 = oracle.dot_w4a16(xb, wc, ws, sgw)
    y44, t44 = oracle.dot_w4a4(ac, as_, sga, wc, ws, sgw, K)
    for m in range(4):
        for n in range(5):
            p = m * 5 + n
            s = sum((F(float(xb[m, k])) * W[n][k] for k in range(K)), F(0))
            t = F(1, 10 ** 5) * sum((abs(F(float(xb[m, k])) * W[n][k]) for k in range(K)), F(0))
            assert abs(F(float(t16[p])) - t) <= tol * t, (m, n)
            assert abs(F(float(y16[p])) - s) <= tol * t * 10 ** 5, (m, n)
            s = sum((A[m][k] * W[n][k] for k in range(K)), F(0))
            t = F(1, 10 ** 5) * sum((abs(A[m][k] * W[n][k]) for k in range(K)), F(0))
            assert abs(F(float(t44[p])) - t) <= tol * t, (m, n)
            assert abs(F(float(y44[p])) - s) <= tol * t * 10 ** 5, (m, n)


def test_matmul_products_agree_with_the_sequential_oracle():
    """The matrix-product form of the W4A4 / W4A16 definitions (float64
    library matmul over the exactly decoded operands) agrees with the
    sequential fp64 dot products to fp64 rounding, at general tensor scales
    and over several 256-wide tiles plus a ragged tail."""
    M, N, K = 37, 300, 1088
    a = inputs.normal_f32((M, K), 81)
    a, _ = inputs.with_outlier_columns(a, 11, 82)
    w = inputs.student_t_f32((N, K), 83)
    ac, as_, sga = oracle.quantize(a)
    wc, ws, sgw = oracle.quantize(w, oracle.MSE)
    y, tau = oracle.dot_w4a4(ac, as_, sga, wc, ws, sgw, K)
    ym, taum = oracle.dot_w4a4_matmul(ac, as_, sga, wc, ws, sgw, K)
    y, tau = y.reshape(M, N), tau.reshape(M, N)
    assert np.all(np.abs(ym - y) <= 1e-12 * tau / 1e-5)
    assert np.allclose(taum, tau, rtol=1e-12, atol=0)
    xb = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(a))
    y16, t16 = oracle.dot_w4a16(xb, wc, ws, sgw)
    y16m, t16m = oracle.dot_w4a16_matmul(xb, wc, ws, sgw)
    y16, t16 = y16.reshape(M, N), t16.reshape(M, N)
    assert np.all(np.abs(y16m - y16) <= 1e-12 * t16 / 1e-5)
    assert np.allclose(t16m, t16, rtol=1e-12, atol=0)


def test_lora_term_numpy_crosscheck_and_tolerance_parts():
    rng = np.random.default_rng(11)
    M, K, r, N = 5, 96, 16, 7
    x = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    A = inputs.bf16_bits_to_f32(inputs.to_bf16_bits((rng.standard_normal((r, K)) * 0.05).astype(np.float32)))
    B = inputs.bf16_bits_to_f32(inputs.to_bf16_bits((rng.standard_normal((N, r)) * 0.05).astype(np.float32)))
    y, tau = oracle.lora_term(x, A, B)
    L = x.astype(np.float64) @ A.astype(np.float64).T
    ref = (L @ B.astype(np.float64).T).reshape(-1)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)
    S = np.abs(x.astype(np.float64)) @ np.abs(A.astype(np.float64)).T
    tref = (np.ldexp(np.abs(L), -8) @ np.abs(B.astype(np.float64)).T + 1e-5 * (S @ np.abs(B.astype(np.float64)).T))
    assert np.allclose(tau, tref.reshape(-1), rtol=1e-12)


def test_lora_term_small_integers_exact_and_zero_branch():
    rng = np.random.default_rng(12)
    x = rng.integers(-4, 5, size=(3, 32)).astype(np.float32)
    A = rng.integers(-3, 4, size=(16, 32)).astype(np.float32)
    B = rng.integers(-2, 3, size=(4, 16)).astype(np.float32)
    y, _ = oracle.lora_term(x, A, B)
    exact_int = (x.astype(np.int64) @ A.astype(np.int64).T) @ B.astype(np.int64).T
    assert np.array_equal(y, exact_int.reshape(-1).astype(np.float64))
    y0, t0 = oracle.lora_term(x, np.zeros_like(A), B)
    assert not y0.any() and not t0.any()


def test_tiny_config_end_to_end_is_consistent():
    w, xb = inputs.tiny()
    codes, scales, sg = oracle.quantize(w)
    assert codes.shape == (256, 128) and scales.shape == (256, 16)
    x = inputs.bf16_bits_to_f32(xb)
    y, tau = oracle.dot_w4a16(x, codes, scales, sg)
    wh = oracle.dequant(codes, scales, sg, 256, 256).astype(np.float64)
    # fp32-rounded dequant vs exact: differences below 2^-23 * sum |x||w^|
    assert np.all(np.abs(y - (x.astype(np.float64) @ wh.T)[0]) <= 2.0 ** -23 * (np.abs(x) @ np.abs(wh).T)[0])


def test_mse_statistics_report():
    """Parity unpinned (the page's ~0.70 x absmax and >25 % claims are narrative):
    reported, not gated; only the invariant E(mse) <= E(absmax) is asserted."""
    w = inputs.student_t_f32((64, 1024), 77)
    ca, sa, sg = oracle.quantize(w, oracle.ABSMAX)
    cm, sm, _ = oracle.quantize(w, oracle.MSE)
    ea = (oracle.dequant(ca, sa, sg, 64, 1024).astype(np.float64) - w) ** 2
    em = (oracle.dequant(cm, sm, sg, 64, 1024).astype(np.float64) - w) ** 2
    ba = ea.reshape(-1, 16).sum(1)
    bm = em.reshape(-1, 16).sum(1)
    assert np.all(bm <= ba * (1 + 1e-6))
    e4 = np.array([oracle.e4m3_value(c) for c in range(127)])
    ratio = e4[sm.reshape(-1)] / np.maximum(e4[sa.reshape(-1)], 1e-30)
    print(f"median s_mse/s_absmax = {np.median(ratio):.3f}; noise variance reduction = "
          f"{1 - em.sum() / ea.sum():.3f}; blocks improved = {(bm < ba).mean():.3f}")


# ---------------------------------------------------------------- static activation scale sweep (R13)

def _e4m3_from_torch(byte):
    return float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)[0])


def test_act_scale_candidates_exact():
    vs = [_e4m3_from_torch(126 - c) for c in range(oracle.SWEEP_CANDIDATES)]
    assert vs[0] == 448.0 and vs[-1] == 112.0 and all(a > b for a, b in zip(vs, vs[1:]))
    g = inputs.rng(31)
    for amax in list(g.uniform(0, 50, 200).astype(np.float32)) + [np.float32(2304.0), np.float32(1e-30)]:
        cand = oracle.act_scale_candidates(amax)
        for c, v in enumerate(vs):
            assert cand[c] == float(exact.fp32(F(float(amax)) / (6 * F(v)))), (amax, c)
        assert cand[0] == oracle.global_scale(float(amax))      # c = 0 is the dynamic rule's s_g
    assert np.all(oracle.act_scale_candidates(0.0) == 1.0)


def _exact_sweep(batches):
    amax = max(float(np.abs(b).max()) for b in batches)
    vs = [F(_e4m3_from_torch(126 - c)) for c in range(oracle.SWEEP_CANDIDATES)]
    errs = []
    for v in vs:
        s = exact.fp32(F(amax) / (6 * v)) if amax > 0 else F(1)
        e = F(0)
        for b in batches:
            for blk in b.reshape(-1, 16):
                bl = [F(float(t)) for t in blk]
                e += exact.block_error(bl, exact.absmax_scale(bl, s), s)
        errs.append(e)
    return errs


def test_act_scale_sweep_matches_exact_rational():
    b1 = _blocks_tiny(41, 8)
    b2 = _blocks_tiny(42, 8) * np.float32(3.0)
    err, best, scale, amax = oracle.act_scale_sweep([b1, b2])
    want = _exact_sweep([b1, b2])
    for c in range(oracle.SWEEP_CANDIDATES):
        assert abs(err[c] - float(want[c])) <= 1e-12 * float(want[c]), c
    exact_best = min(range(oracle.SWEEP_CANDIDATES), key=lambda c: (want[c], c))
    assert best == exact_best
    assert scale == oracle.act_scale_candidates(amax)[best]


def test_act_scale_sweep_constructed_winner():
    """amax = 6 * 384: candidate 2 (v = 384) gives s = 1 exactly, under which
    both blocks lie on their grids (scales 384 and 1), so its error is exactly
    zero; the dynamic rule's s_g = fp32(2304 / 2688) rounds and cannot."""
    blk1 = np.array([2304, -1152, 576, 192, 0, 384, -768, 1536, 1152, -2304, 96 * 2, 0, 576, -192, 384, 768],
                    dtype=np.float32)
    blk2 = np.array([6, -3, 1.5, 0.5, 1, -2, 4, 0, -6, 3, 2, -1, 0.5, -0.5, 1.5, 4], dtype=np.float32)
    err, best, scale, amax = oracle.act_scale_sweep([np.concatenate([blk1, blk2])])
    assert amax == 2304.0 and best == 2 and scale == 1.0
    assert err[2] == 0.0 and err[0] > 0 and err[1] > 0
    want = _exact_sweep([np.concatenate([blk1, blk2])])
    assert want[2] == 0 and all(want[c] > 0 for c in (0, 1))


def test_act_scale_sweep_accumulates_batches_in_order():
    b1 = _blocks_tiny(43, 12)
    b2 = _blocks_tiny(44, 12) * np.float32(0.5)
    e12, best12, _, amax = oracle.act_scale_sweep([b1, b2])
    ecat, bestcat, _, _ = oracle.act_scale_sweep([np.concatenate([b1.reshape(-1), b2.reshape(-1)])])
    assert np.array_equal(e12, ecat) and best12 == bestcat
    e1, _, _, _ = oracle.act_scale_sweep([b1], amax=amax)
    assert np.all(e1 < e12)                      # the second batch adds its own error


def test_act_scale_sweep_zero_input():
    err, best, scale, amax = oracle.act_scale_sweep([np.zeros((4, 32), dtype=np.float32)])
    assert amax == 0.0 and best == 0 and scale == 1.0 and np.all(err == 0)


# ---------------------------------------------------------------- SVDQuant smoothing (R14)

def _fp32_neighbours(v):
    v = np.float32(v)
    return np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(np.inf))


def test_smooth_factors_are_correctly_rounded_sqrt():
    g = inputs.rng(51)
    a = np.concatenate([g.uniform(0, 100, 3000), [4.0, 9.0, 0.0, 5.0, 1e-30, 3.0e30]]).astype(np.float32)
    w = np.concatenate([g.uniform(0, 0.5, 3000), [1.0, 1.0, 2.0, 0.0, 1e-30, 1e-30]]).astype(np.float32)
    lam, mult = oracle.smooth_factors(a, w)
    assert lam[-6] == 2.0 and lam[-5] == 3.0 and lam[-4] == 1.0 and lam[-3] == 1.0 and lam[-2] == 1.0
    for k in range(a.size):
        if a[k] == 0 or w[k] == 0:
            assert lam[k] == 1.0 and mult[k] == 1.0
            continue
        q = F(float(a[k])) / F(float(w[k]))
        lo, hi = _fp32_neighbours(lam[k])
        # lambda is the nearest fp32 to sqrt(q): q lies between the squares of the midpoints
        assert (F(float(lo)) + F(float(lam[k]))) ** 2 / 4 <= q <= (F(float(hi)) + F(float(lam[k]))) ** 2 / 4, k
        assert mult[k] == float(exact.fp32(1 / F(float(lam[k])))), k


def test_smooth_act_exact_and_torch():
    g = inputs.rng(52)
    x = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(g.standard_normal((7, 64)).astype(np.float32) * 3))
    mult = g.uniform(0.01, 20, 64).astype(np.float32)
    got = oracle.smooth_act(x, mult)
    bf16_max = F(2 ** 8 - 1, 2 ** 7) * 2 ** 127
    for m in range(x.shape[0]):
        for k in range(x.shape[1]):
            p = exact.fp32(F(float(x[m, k])) * F(float(mult[k])))
            assert got[m, k] == float(exact.round_format(p, 7, -126, bf16_max)), (m, k)
    want = (torch.from_numpy(x) * torch.from_numpy(mult)).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got, want)
    # a power-of-two multiplier only moves the exponent of a bf16 value
    assert np.array_equal(oracle.smooth_act(x, np.full(64, 0.25, np.float32)), x * np.float32(0.25))
