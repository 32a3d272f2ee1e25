"""GPU parity of the quantizers and the dequantizer against the CPU oracle:
codes, scale bytes and the per-tensor scale must be bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from dit_quantization_amd import inputs
from dit_quantization_amd import nvfp4 as nv
from tests.gpu_helpers import DEV, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


def _gpu_quant(method, x_dev, sg=None):
    fn = {oracle.ABSMAX: nv.quantize_absmax, oracle.MSE: nv.quantize_mse,
          oracle.FOUR_OVER_SIX: nv.quantize_4o6}[method]
    c, s, g = fn(x_dev, global_scale=sg)
    torch.cuda.synchronize()
    return host(c), host(s), float(host(g)[0])


def _check(method, x_f32, x_dev, sg=None, what=""):
    print(f"[case] {what} method={method} shape={x_f32.shape} sg={sg}", flush=True)
    oc, os_, og = oracle.quantize(x_f32, method, sg=sg)
    gc, gs, gg = _gpu_quant(method, x_dev, sg)
    assert gg == og, (what, gg, og)
    assert np.array_equal(gs, os_), (what, np.argwhere(gs != os_)[:5])
    assert np.array_equal(gc, oc), (what, np.argwhere(gc != oc)[:5])


def _adversarial(rows, cols, seed):
    g = inputs.rng(seed)
    x = (g.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    x[0, :16] = 0.0                                            # all-zero block
    if rows > 1:
        x[1, :] *= 1e-6                                        # tiny blocks (subnormal E4M3 scales)
    if rows > 2:
        x[2, ::16] *= 30.0                                     # one outlier per block
    if rows > 3:
        x[3, :] = np.exp(g.uniform(-40, 3, cols)) * g.choice([-1, 1], cols)   # huge dynamic range
    return x


SHAPES = [(1, 32), (3, 96), (37, 160), (129, 4096), (5, 14336)]


@pytest.mark.parametrize("method", [oracle.ABSMAX, oracle.MSE, oracle.FOUR_OVER_SIX])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_fp32_random_shapes(method, shape):
    x = _adversarial(*shape, seed=shape[0] * 7 + shape[1])
    _check(method, x, dev_f32(x), what=f"fp32 {shape}")


@pytest.mark.parametrize("method", [oracle.ABSMAX, oracle.MSE, oracle.FOUR_OVER_SIX])
@pytest.mark.parametrize("shape", [(2, 64), (33, 480), (64, 3072)])
def test_quantize_bf16(method, shape):
    a = inputs.normal_f32(shape, 100 + shape[0])
    a, _ = inputs.with_outlier_columns(a, max(1, shape[1] // 100), 5)
    bits = inputs.to_bf16_bits(a)
    _check(method, inputs.bf16_bits_to_f32(bits), dev_bf16(bits), what=f"bf16 {shape}")


@pytest.mark.parametrize("method", [oracle.ABSMAX, oracle.MSE, oracle.FOUR_OVER_SIX])
@pytest.mark.parametrize("sg", [1.0, 1e-3, 37.5, 1e-30])
def test_quantize_given_global_scale(method, sg):
    x = _adversarial(8, 256, seed=int(sg * 1000) % 97)
    _check(method, x, dev_f32(x), sg=sg, what=f"given sg {sg}")


@pytest.mark.parametrize("method", [oracle.ABSMAX, oracle.MSE, oracle.FOUR_OVER_SIX])
def test_quantize_exact_ties(method):
    # s_g = 1 given; elements on every E2M1 midpoint of several scales, and
    # block maxima on E4M3 midpoints
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    rows = []
    for c in (1, 8, 20, 56, 100, 125, 126):
        sb = e4[c]
        mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
        rows.append([6 * sb] + [m * sb for m in mids] + [-m * sb for m in mids] + [0.0] +
                    [m * sb * (1 + 2 ** -20) for m in mids] + [-m * sb * (1 - 2 ** -20) for m in mids] + [0.0, 0.0])
    for lo, hi in zip(e4[1:-1:3], e4[2::3]):
        mid = (lo + hi) / 2
        rows.append([6 * mid] + [0.3 * mid] * 15 + [-6 * mid] + [1.7 * mid] * 15)
    x = np.array(rows, dtype=np.float32)
    _check(method, x, dev_f32(x), sg=1.0, what="ties")


def test_dequant_exhaustive_codes_and_scales():
    # row r: every code byte 0..255 once, every block scaled by E4M3 byte r
    codes = np.tile(np.arange(256, dtype=np.uint8), (127, 1))
    scales = np.repeat(np.arange(127, dtype=np.uint8)[:, None], 32, axis=1)
    for sg in (1.0, 0.3712, 5e-3):
        ref = oracle.dequant(codes, scales, sg, 127, 512)
        gsg = torch.tensor([sg], dtype=torch.float32, device=DEV)
        out32 = host(nv.dequant(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), gsg))
        assert np.array_equal(out32.view(np.uint32), ref.view(np.uint32)), sg
        outb = host(nv.dequant(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), gsg,
                               out_dtype=torch.bfloat16))
        refb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(outb, refb), sg


def test_tiny_config_quantize():
    w, _ = inputs.tiny()
    _check(oracle.ABSMAX, w, dev_f32(w), what="tiny 256x256")


@pytest.mark.parametrize("method", [oracle.MSE, oracle.FOUR_OVER_SIX])
@pytest.mark.parametrize("name", ["q", "k", "down"])
def test_layerset_search_full_size_sampled_rows(name, method):
    (_, w), = list(inputs.layerset([name]))
    print(f"[case] layerset {name} {w.shape} method {method}", flush=True)
    gc, gs, gg = _gpu_quant(method, dev_f32(w))
    sg = oracle.global_scale(float(np.abs(w).max()))
    assert gg == sg
    rows = np.unique(np.concatenate([[0, w.shape[0] - 1], inputs.rng(5).choice(w.shape[0], 48, replace=False)]))
    oc, os_, _ = oracle.quantize(w[rows], method, sg=sg)
    assert np.array_equal(gs[rows], os_)
    assert np.array_equal(gc[rows], oc)


def test_quantize_is_deterministic():
    w = inputs.student_t_f32((512, 1024), 9)
    xd = dev_f32(w)
    a = _gpu_quant(oracle.MSE, xd)
    b = _gpu_quant(oracle.MSE, xd)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


@pytest.mark.parametrize("offset", [1, 2, 3])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_quantize_absmax_unaligned_scales(offset, dtype):
    """The absmax pass stores four scale bytes per dword store when the scales
    buffer is 4-byte aligned; a caller's buffer at any other offset takes the
    byte stores, with the same result."""
    rows, cols = 37, 160
    x = _adversarial(rows, cols, seed=offset + 17)
    if dtype == "bf16":
        bits = inputs.to_bf16_bits(x)
        x, xd = inputs.bf16_bits_to_f32(bits), dev_bf16(bits)
    else:
        xd = dev_f32(x)
    print(f"[case] absmax {dtype} scales at byte offset {offset}", flush=True)
    oc, os_, og = oracle.quantize(x, oracle.ABSMAX)
    buf = torch.full((rows * cols // 16 + 8,), 0xEE, dtype=torch.uint8, device=DEV)
    scales = buf[offset:offset + rows * cols // 16].view(rows, cols // 16)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
    sg = torch.empty(1, dtype=torch.float32, device=DEV)
    nv.quantize_absmax(xd, out=(codes, scales, sg))
    torch.cuda.synchronize()
    assert float(host(sg)[0]) == og
    assert np.array_equal(host(codes), oc)
    assert np.array_equal(host(scales), os_)
    b = host(buf)
    assert np.all(b[:offset] == 0xEE) and np.all(b[offset + rows * cols // 16:] == 0xEE)   # nothing written outside


def test_quantize_empty_tensor():
    """An empty tensor quantizes to empty codes and scales; a computed tensor
    scale is 1.0 (zero amax), a given one is left as it is."""
    print("[case] quantize empty tensor", flush=True)
    for fn in (nv.quantize_absmax, nv.quantize_mse, nv.quantize_4o6):
        c, s, g = fn(torch.empty((0, 64), dtype=torch.float32, device="cuda:0"))
        assert c.shape == (0, 32) and s.shape == (0, 4) and float(g.item()) == 1.0
        c, s, g = fn(torch.empty((3, 0), dtype=torch.bfloat16, device="cuda:0"),
                     global_scale=torch.tensor([0.25], device="cuda:0"))
        assert c.shape == (3, 0) and s.shape == (3, 0) and float(g.item()) == 0.25
