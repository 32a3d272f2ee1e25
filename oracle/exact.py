"""Exact-rational NVFP4 checker -- TEST INFRASTRUCTURE ONLY.

An independent second implementation of the quantizer contract for tiny
inputs, in Python `fractions` (no floating point in any decision).  Where the
C oracle finds nearest values by an argmin over an enumerated grid, this
module rounds to a binary floating-point *format* (significand bits, minimum
exponent, saturation), so the two agree only if both are right.

Formats: E2M1 = 1 fraction bit, minimum exponent 0 (subnormal step 0.5),
largest value 6 ("Tu pipeline NVFP4 ...", section 2, the E2M1 bitfield
formula); E4M3 = 3 fraction bits, minimum exponent -6, largest finite 448
(float8_e4m3fn); fp32 = 23 fraction bits, minimum exponent -126.
"""
from fractions import Fraction as F

E4M3_MAX = F(448)
E2M1_MAX = F(6)
FP32_MAX = F(2 ** 24 - 1, 2 ** 23) * 2 ** 127


def floor_log2(a: F) -> int:
    """e with 2^e <= a < 2^(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    elif F(2) ** (e + 1) <= a:
        e += 1
    return e


def round_format(x: F, frac_bits: int, emin: int, maxval: F, saturate: bool = True) -> F:
    """Nearest value of the binary format to x; exact ties go to the even
    significand; magnitudes beyond maxval saturate (or raise)."""
    if x == 0:
        return F(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(floor_log2(a), emin)
    quantum = F(2) ** (e - frac_bits)
    n = a / quantum
    r = round(n)                # Fraction.__round__: half to even
    val = r * quantum
    if val > maxval:
        if not saturate:
            raise OverflowError(x)
        val = maxval
    return sign * val


def fp32(x: F) -> F:
    return round_format(x, 23, -126, FP32_MAX, saturate=False)


def e4m3_values():
    """All non-negative finite E4M3 values, ascending (index = byte code)."""
    vals = [F(m, 8) * F(2) ** -6 for m in range(8)]                       # subnormals
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                                   # NaN
            vals.append((1 + F(m, 8)) * F(2) ** (e - 7))
    return vals


E4M3 = e4m3_values()
E4M3_INDEX = {v: i for i, v in enumerate(E4M3)}
E2M1_MAG = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def e2m1_code(value: F) -> int:
    if value == 0:
        return 0
    idx = E2M1_MAG.index(abs(value))
    return idx | (8 if value < 0 else 0)


def global_scale(amax) -> F:
    amax = F(amax)
    if amax == 0:
        return F(1)
    return fp32(amax / 2688)


def absmax_scale(block, sg) -> F:
    a = max(abs(F(w)) for w in block) / (6 * F(sg))
    return round_format(a, 3, -6, E4M3_MAX)


def codes_for(block, sb: F, sg) -> list:
    if sb == 0:
        return [0] * len(block)
    d = sb * F(sg)
    return [e2m1_code(round_format(F(w) / d, 1, 0, E2M1_MAX)) for w in block]


def recon(block, sb: F, sg) -> list:
    cs = codes_for(block, sb, sg)
    out = []
    for c in cs:
        mag = E2M1_MAG[c & 7]
        out.append(-mag * sb * F(sg) if c & 8 else mag * sb * F(sg))
    return out


def block_error(block, sb: F, sg) -> F:
    return sum(((F(w) - r) ** 2 for w, r in zip(block, recon(block, sb, sg))), F(0))


def mse_search(block, sg):
    """Exact MSE search.  Returns (windowed choice, its error, global argmin
    over all non-negative E4M3 scales, its error).  The windowed set is the
    positive E4M3 values in [a/2, min(2a, 448)] plus the absmax scale; ties
    keep the smaller scale."""
    a = max(abs(F(w)) for w in block) / (6 * F(sg))
    sabs = round_format(a, 3, -6, E4M3_MAX)
    best = best_err = None
    gbest = gbest_err = None
    for v in E4M3:
        err = block_error(block, v, sg)
        if gbest is None or err < gbest_err:
            gbest, gbest_err = v, err
        in_window = v > 0 and a / 2 <= v <= 2 * a
        if in_window or v == sabs:
            if best is None or err < best_err:
                best, best_err = v, err
    return best, best_err, gbest, gbest_err


def four_over_six(block, sg):
    """Exact four-over-six choice: the E4M3 roundings of max|W| / (6 s_g) and
    max|W| / (4 s_g); the smaller exact error wins and a tie keeps the
    smaller scale.  Returns (scale, error)."""
    m = max(abs(F(w)) for w in block)
    c6 = round_format(m / (6 * F(sg)), 3, -6, E4M3_MAX)
    c4 = round_format(m / (4 * F(sg)), 3, -6, E4M3_MAX)
    e6 = block_error(block, c6, sg)
    e4 = block_error(block, c4, sg)
    return (c4, e4) if e4 < e6 else (c6, e6)
