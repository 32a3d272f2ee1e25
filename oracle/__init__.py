"""NVFP4 reference oracle -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The GPU library never imports, links or calls it, and
this package never touches the GPU library.  It wraps the plain C oracle
(nvfp4_oracle.c, fp64, no FMA contraction) with numpy marshalling only:
every numeric decision is taken in the C code.  `exact.py` is a second,
independent checker in exact rational arithmetic for tiny inputs.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ABSMAX = 0
MSE = 1
FOUR_OVER_SIX = 2


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(
            os.path.join(_HERE, "nvfp4_oracle.c")):
        from . import build_oracle
        build_oracle.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
    lib.oracle_e4m3_nearest.restype = ctypes.c_int
    lib.oracle_e4m3_nearest.argtypes = [ctypes.c_double]
    lib.oracle_e2m1_nearest.restype = ctypes.c_int
    lib.oracle_e2m1_nearest.argtypes = [ctypes.c_double]
    lib.oracle_amax.restype = ctypes.c_float
    lib.oracle_amax.argtypes = [P, i64]
    lib.oracle_global_scale.restype = ctypes.c_float
    lib.oracle_global_scale.argtypes = [ctypes.c_float]
    lib.oracle_absmax_scale_code.restype = ctypes.c_int
    lib.oracle_absmax_scale_code.argtypes = [P, ctypes.c_float]
    lib.oracle_mse_scale_code.restype = ctypes.c_int
    lib.oracle_mse_scale_code.argtypes = [P, ctypes.c_float]
    lib.oracle_lora_term.restype = ctypes.c_int
    lib.oracle_lora_term.argtypes = [P, P, P, i64, i64, P, P, i64, P, P, ctypes.c_int]
    lib.oracle_act_scale_errors.restype = ctypes.c_int
    lib.oracle_act_scale_errors.argtypes = [P, i64, ctypes.c_float, P, ctypes.c_int]
    lib.oracle_smooth_factors.restype = None
    lib.oracle_smooth_factors.argtypes = [P, P, i64, P, P]
    lib.oracle_smooth_act.restype = None
    lib.oracle_smooth_act.argtypes = [P, P, i64, i64, P]
    lib.oracle_4o6_scale_code.restype = ctypes.c_int
    lib.oracle_4o6_scale_code.argtypes = [P, ctypes.c_float]
    lib.oracle_block_error.restype = ctypes.c_double
    lib.oracle_block_error.argtypes = [P, ctypes.c_float, ctypes.c_int]
    lib.oracle_quantize.restype = ctypes.c_int
    lib.oracle_quantize.argtypes = [ctypes.c_int, P, i64, i64, ctypes.c_int, P, P, P, ctypes.c_int]
    lib.oracle_dequant.restype = ctypes.c_int
    lib.oracle_dequant.argtypes = [P, P, ctypes.c_float, i64, i64, P]
    lib.oracle_dot_w4a16.restype = ctypes.c_int
    lib.oracle_dot_w4a16.argtypes = [P, P, P, ctypes.c_float, i64, P, P, i64, P, P, ctypes.c_int]
    lib.oracle_dot_w4a4.restype = ctypes.c_int
    lib.oracle_dot_w4a4.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, i64, P, P, i64, P, P,
                                    ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _threads(threads):
    if threads is None:
        return len(os.sched_getaffinity(0))
    return int(threads)


def e2m1_value(code):
    return _load().oracle_e2m1_value(int(code))


def e4m3_value(byte):
    return _load().oracle_e4m3_value(int(byte))


def e4m3_nearest(a):
    return _load().oracle_e4m3_nearest(float(a))


def e2m1_nearest(x):
    return _load().oracle_e2m1_nearest(float(x))


def global_scale(amax):
    return float(np.float32(_load().oracle_global_scale(float(np.float32(amax)))))


def _as_f32_2d(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    return x


def absmax_scale_code(block, sg):
    b = np.ascontiguousarray(block, dtype=np.float32).reshape(16)
    return _load().oracle_absmax_scale_code(_ptr(b), float(np.float32(sg)))


def mse_scale_code(block, sg):
    b = np.ascontiguousarray(block, dtype=np.float32).reshape(16)
    return _load().oracle_mse_scale_code(_ptr(b), float(np.float32(sg)))


def four_over_six_scale_code(block, sg):
    b = np.ascontiguousarray(block, dtype=np.float32).reshape(16)
    return _load().oracle_4o6_scale_code(_ptr(b), float(np.float32(sg)))


def block_error(block, sg, scale_code):
    b = np.ascontiguousarray(block, dtype=np.float32).reshape(16)
    return _load().oracle_block_error(_ptr(b), float(np.float32(sg)), int(scale_code))


def quantize(x, method=ABSMAX, sg=None, threads=None):
    """Quantize a [rows, cols] float32 array (bf16 data widened to fp32).

    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], sg float).
    sg=None computes the per-tensor scale; a number uses it as given.
    """
    x = _as_f32_2d(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    sgv = np.zeros(1, dtype=np.float32)
    given = sg is not None
    if given:
        sgv[0] = np.float32(sg)
    rc = _load().oracle_quantize(int(method), _ptr(x), rows, cols, int(given), _ptr(sgv), _ptr(codes),
                                 _ptr(scales), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_quantize: bad shape %r" % (x.shape,))
    return codes, scales, float(sgv[0])


def dequant(codes, scales, sg, rows, cols):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.zeros((rows, cols), dtype=np.float32)
    rc = _load().oracle_dequant(_ptr(codes), _ptr(scales), float(np.float32(sg)), rows, cols, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequant: bad shape")
    return out


def _pairs(M, N, pairs):
    if pairs is None:
        pm, pn = np.meshgrid(np.arange(M, dtype=np.int64), np.arange(N, dtype=np.int64), indexing="ij")
        return pm.reshape(-1).copy(), pn.reshape(-1).copy()
    pm = np.ascontiguousarray(pairs[0], dtype=np.int64)
    pn = np.ascontiguousarray(pairs[1], dtype=np.int64)
    return pm, pn


def dot_w4a16(x, w_codes, w_scales, sgw, pairs=None, N=None, threads=None):
    """fp64 y*[m,n] and tau for the requested (m, n) pairs (all pairs if None)."""
    x = _as_f32_2d(x)
    M, K = x.shape
    if N is None:
        N = w_scales.shape[0]
    pm, pn = _pairs(M, N, pairs)
    y = np.zeros(pm.shape[0], dtype=np.float64)
    tau = np.zeros(pm.shape[0], dtype=np.float64)
    wc = np.ascontiguousarray(w_codes, dtype=np.uint8)
    ws = np.ascontiguousarray(w_scales, dtype=np.uint8)
    rc = _load().oracle_dot_w4a16(_ptr(x), _ptr(wc), _ptr(ws), float(np.float32(sgw)), K, _ptr(pm), _ptr(pn),
                                  pm.shape[0], _ptr(y), _ptr(tau), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_dot_w4a16: bad shape")
    return y, tau


def dot_w4a4(a_codes, a_scales, sga, w_codes, w_scales, sgw, K, pairs=None, M=None, N=None, threads=None):
    """fp64 y*[m,n] and tau for NVFP4 x NVFP4 operands (all pairs if None)."""
    if M is None:
        M = a_scales.shape[0]
    if N is None:
        N = w_scales.shape[0]
    pm, pn = _pairs(M, N, pairs)
    y = np.zeros(pm.shape[0], dtype=np.float64)
    tau = np.zeros(pm.shape[0], dtype=np.float64)
    ac = np.ascontiguousarray(a_codes, dtype=np.uint8)
    as_ = np.ascontiguousarray(a_scales, dtype=np.uint8)
    wc = np.ascontiguousarray(w_codes, dtype=np.uint8)
    ws = np.ascontiguousarray(w_scales, dtype=np.uint8)
    rc = _load().oracle_dot_w4a4(_ptr(ac), _ptr(as_), float(np.float32(sga)), _ptr(wc), _ptr(ws),
                                 float(np.float32(sgw)), K, _ptr(pm), _ptr(pn), pm.shape[0], _ptr(y), _ptr(tau),
                                 _threads(threads))
    if rc != 0:
        raise ValueError("oracle_dot_w4a4: bad shape")
    return y, tau


def dot_w4a4_matmul(a_codes, a_scales, sga, w_codes, w_scales, sgw, K):
    """y* and tau for every (m, n) of the given operand rows, by the same
    definition as dot_w4a4 ("NVFP4 en difusion ...", section 2: out =
    (A s_a)(B s_b)^T; fp64 sums, tau = 1e-5 sum_k |a^||w^|), with a float64
    matrix product (a library primitive) taking the K-sums.  The operands
    are the oracle's dequant at s_g = 1: the exact values q s_b (at most 6
    significant bits, magnitudes 2^-10 .. 2688, exact in fp32); every product
    is exact in fp64 and the exact fp64 product s_gA s_gW scales the sums.
    Only the order of the fp64 additions differs from dot_w4a4, which keeps
    the two within about K 2^-53 sum |a^||w^| of each other."""
    M, N = a_scales.shape[0], w_scales.shape[0]
    A = dequant(a_codes, a_scales, 1.0, M, K).astype(np.float64)
    W = dequant(w_codes, w_scales, 1.0, N, K).astype(np.float64)
    g = float(np.float32(sga)) * float(np.float32(sgw))
    y = (A @ W.T) * g
    tau = 1e-5 * ((np.abs(A) @ np.abs(W).T) * g)
    return y, tau


def dot_w4a16_matmul(x, w_codes, w_scales, sgw):
    """W4A16 counterpart of dot_w4a4_matmul: y* = s_gW x (q_w s_w)^T and
    tau = 1e-5 |x| |w^|^T for bf16 x [M, K] given as float32 (products of
    a bf16 and a q s_b value have at most 14 significant bits: exact)."""
    x = _as_f32_2d(x).astype(np.float64)
    N = w_scales.shape[0]
    W = dequant(w_codes, w_scales, 1.0, N, x.shape[1]).astype(np.float64)
    g = float(np.float32(sgw))
    return (x @ W.T) * g, 1e-5 * ((np.abs(x) @ np.abs(W).T) * g)


def lora_term(x, A, B, pairs=None, threads=None):
    """fp64 low-rank term y*_L[m,n] = sum_j (x A^T)[m,j] B[n,j] and its
    tolerance for the requested (m, n) pairs (all pairs if None).  x [M, K],
    A [r, K], B [N, r]: 16-bit values as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    M, K = x.shape
    r = A.shape[0]
    N = B.shape[0]
    if A.shape != (r, K) or B.shape != (N, r):
        raise ValueError("lora_term: shapes must be x [M, K], A [r, K], B [N, r]")
    pm, pn = _pairs(M, N, pairs)
    y = np.zeros(pm.shape[0], dtype=np.float64)
    tau = np.zeros(pm.shape[0], dtype=np.float64)
    rc = _load().oracle_lora_term(_ptr(x), _ptr(A), _ptr(B), r, K, _ptr(pm), _ptr(pn), pm.shape[0], _ptr(y),
                                  _ptr(tau), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_lora_term: bad shape")
    return y, tau


SWEEP_CANDIDATES = 17


def act_scale_candidates(amax):
    """Candidate static activation tensor scales s_c = fp32(amax / (6 v_c)),
    v_c = E4M3(126 - c) = 448 ... 112 (all 1.0 when amax == 0); reading R13."""
    lib = _load()
    if np.float32(amax) == 0:
        return np.ones(SWEEP_CANDIDATES, dtype=np.float32)
    return np.array([np.float32(np.float64(np.float32(amax)) / (6.0 * lib.oracle_e4m3_value(126 - c)))
                     for c in range(SWEEP_CANDIDATES)], dtype=np.float32)


def act_scale_sweep(batches, amax=None, threads=None):
    """FP8 candidate sweep for a static activation tensor scale over calibration
    batches (each any shape with a multiple of 16 elements per row-major
    block run).  Returns (errors fp64 [17], best index, chosen scale fp32,
    amax): errors accumulate over the batches in order, the smallest error
    wins and ties keep the lower index."""
    batches = [np.ascontiguousarray(b, dtype=np.float32).reshape(-1) for b in batches]
    if amax is None:
        amax = max((float(_load().oracle_amax(_ptr(b), b.size)) for b in batches), default=0.0)
    amax = np.float32(amax)
    err = np.zeros(SWEEP_CANDIDATES, dtype=np.float64)
    for b in batches:
        if _load().oracle_act_scale_errors(_ptr(b), b.size, amax, _ptr(err), _threads(threads)) != 0:
            raise ValueError("act_scale_sweep: a batch's size is not a multiple of 16")
    best = 0
    for c in range(1, SWEEP_CANDIDATES):
        if err[c] < err[best]:
            best = c
    return err, best, act_scale_candidates(amax)[best], amax


def smooth_factors(act_amax, w_amax):
    """SVDQuant per-channel smoothing (reading R14): (lambda, mult) fp32 [K],
    lambda_k = fp32(sqrt(a_k / w_k)) (1 if either is 0), mult_k = fp32(1 / lambda_k)."""
    a = np.ascontiguousarray(act_amax, dtype=np.float32)
    w = np.ascontiguousarray(w_amax, dtype=np.float32)
    if a.shape != w.shape or a.ndim != 1:
        raise ValueError("smooth_factors: two [K] vectors")
    lam = np.empty_like(a)
    mult = np.empty_like(a)
    _load().oracle_smooth_factors(_ptr(a), _ptr(w), a.size, _ptr(lam), _ptr(mult))
    return lam, mult


def smooth_act(x, mult):
    """x^ = bf16(fp32(x * mult)) per input channel, as float32 [M, K]."""
    x = _as_f32_2d(x)
    mult = np.ascontiguousarray(mult, dtype=np.float32)
    M, K = x.shape
    if mult.shape != (K,):
        raise ValueError("smooth_act: mult must be [K]")
    out = np.empty_like(x)
    _load().oracle_smooth_act(_ptr(x), _ptr(mult), M, K, _ptr(out))
    return out


def bf16_rne_from_f64(v):
    """Round fp64 values to the nearest bfloat16 value (ties to even), exactly,
    returned as fp64.  Used for the output bracket of a bf16 GEMM result."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # bf16 subnormal spacing 2^-133
    scaled = np.ldexp(v, 8 - e)             # 8 significant bits kept
    return np.ldexp(np.rint(scaled), e - 8)


def bracket_bf16(y, tau):
    """Pass interval [bf16(y*-tau), bf16(y*+tau)] for a bf16 output."""
    return bf16_rne_from_f64(np.asarray(y) - np.asarray(tau)), bf16_rne_from_f64(np.asarray(y) + np.asarray(tau))
