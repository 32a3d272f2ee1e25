"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers (numpy PCG64) with the shapes and value
distributions of the workloads; it holds none of the quantizer's or GEMM's
arithmetic.  Both the GPU library and the CPU oracle are fed from here.

Workloads (weights "approximately Gaussian" or heavy-tailed Student-t,
activations with ~1 % outlier channels at 20x, standing in for real
checkpoints and calibration data that are not available):
  tiny      W [256, 256] ~ N(0, 0.02^2) seed 0; x [1, 256] ~ N(0, 1) bf16
  gemv      W1 [14336, 4096] seed 1, W2 [4096, 14336] seed 2 ~ N(0, 0.02^2);
            x [16, K] ~ N(0, 1) bf16 seed 3 (M = 1, 4 use the first rows)
  layerset  8B-shaped set q, o [4096, 4096]; k, v [1024, 4096];
            gate, up [14336, 4096]; down [4096, 14336]; t(5) * 0.02, seeds 10..16
  prefill   A [4096, 4096] ~ N(0, 1) seed 20, 41 outlier columns (seed 21) x20, bf16;
            W = layerset gate [14336, 4096]
  dit       Flux-like double-stream block, hidden 3072, MLP 12288, image M = 4096,
            text M = 512; weights t(5) * 0.02 seeds 30..39; activations N(0, 1)
            with 1 % x20 outlier columns, seeds 40..43
  lora      low-rank factors of rank r (tens): down [r, K] ~ N(0, 1/K),
            up [N, r] ~ N(0, 0.03^2), bf16; a trained correction of about a
            tenth of the layer output at r = 32
"""
import numpy as np

LAYERSET = [  # name, (rows, cols), seed
    ("q", (4096, 4096), 10),
    ("k", (1024, 4096), 11),
    ("v", (1024, 4096), 12),
    ("o", (4096, 4096), 13),
    ("gate", (14336, 4096), 14),
    ("up", (14336, 4096), 15),
    ("down", (4096, 14336), 16),
]

DIT_WEIGHTS = [  # name, (out, in)
    ("to_q", (3072, 3072)),
    ("to_k", (3072, 3072)),
    ("to_v", (3072, 3072)),
    ("mlp_up", (12288, 3072)),
    ("mlp_down", (3072, 12288)),
]


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(shape, seed, std=1.0):
    g = rng(seed)
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def student_t_f32(shape, seed, df=5, scale=0.02):
    g = rng(seed)
    return (g.standard_t(df, size=shape) * scale).astype(np.float32)


def to_bf16_bits(x_f32):
    """bf16 storage of fp32 data (round to nearest even), as uint16 bit patterns."""
    u = np.ascontiguousarray(x_f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def with_outlier_columns(a_f32, n_out, seed, factor=20.0):
    """Scale n_out randomly chosen columns (activation channels) by `factor`."""
    cols = rng(seed).choice(a_f32.shape[1], n_out, replace=False)
    a_f32[:, cols] *= np.float32(factor)
    return a_f32, np.sort(cols)


def tiny():
    g = rng(0)
    w = (g.standard_normal((256, 256)) * 0.02).astype(np.float32)
    x = g.standard_normal((1, 256)).astype(np.float32)
    return w, to_bf16_bits(x)


def gemv_weights():
    return normal_f32((14336, 4096), 1, 0.02), normal_f32((4096, 14336), 2, 0.02)


def gemv_x(K, M=16):
    return to_bf16_bits(normal_f32((M, K), 3))


def layerset(names=None):
    for name, shape, seed in LAYERSET:
        if names is None or name in names:
            yield name, student_t_f32(shape, seed)


def prefill_activation():
    a = normal_f32((4096, 4096), 20)
    a, _ = with_outlier_columns(a, 41, 21)
    return to_bf16_bits(a)


def dit_weights(stream):
    """stream 0 = image, 1 = text; five matrices each, seeds 30..39."""
    base = 30 + 5 * stream
    return [(name, student_t_f32(shape, base + i)) for i, (name, shape) in enumerate(DIT_WEIGHTS)]


def dit_activations():
    """(A_img [4096,3072], A_txt [512,3072], H_img [4096,12288], H_txt [512,12288]) bf16 bits."""
    out = []
    for seed, (m, k) in zip((40, 41, 42, 43), ((4096, 3072), (512, 3072), (4096, 12288), (512, 12288))):
        a = normal_f32((m, k), seed)
        a, _ = with_outlier_columns(a, max(1, k // 100), seed + 100)
        out.append(to_bf16_bits(a))
    return tuple(out)


def lora_factors(r, K, N, seed, up_std=0.03):
    """(down [r, K], up [N, r]) bf16 bits of a rank-r LoRA branch."""
    down = normal_f32((r, K), seed, std=1.0 / np.sqrt(K))
    up = normal_f32((N, r), seed + 1, std=up_std)
    return to_bf16_bits(down), to_bf16_bits(up)


def random_bf16_bits(shape, seed):
    """bf16 bit patterns with a random sign, a random 7-bit mantissa and one
    of four exponents (magnitudes in [1/8, 4)): every element random, drawn
    in row chunks so large edge-case operands stay cheap to make."""
    g = rng(seed)
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    step = max(1, (1 << 26) // max(1, int(np.prod(shape[1:]))))
    for r0 in range(0, rows, step):
        r = g.integers(0, 1 << 16, size=(min(step, rows - r0),) + tuple(shape[1:]), dtype=np.uint16)
        o = out[r0:r0 + r.shape[0]]
        np.bitwise_and(r, 0x807F, out=o)        # sign and mantissa
        r >>= 7
        r &= 3
        r += 124                                # exponent 124 .. 127
        r <<= 7
        o |= r
    return out


def random_nvfp4_weight(rows, cols, seed):
    """An NVFP4 weight made of random code bytes, random E4M3 scale bytes in
    0x28..0x47 (0.125 .. 1.875) and a tensor scale 1/2688: (codes [rows,
    cols/2] u8, scales [rows, cols/16] u8, s_g)."""
    g = rng(seed)
    codes = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = g.integers(0x28, 0x48, size=(rows, cols // 16), dtype=np.uint8)
    return codes, scales, float(np.float32(1.0 / 2688.0))
