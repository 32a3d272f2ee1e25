"""SVDQuant weight preparation for the fused low-rank W4A4 layer.

"NVFP4 en difusion: la misma cuantizacion, un motor completamente distinto",
section 3: SVDQuant first moves the activation outliers into the weights by
scaling each input channel, then splits the scaled weights into a 16-bit
low-rank part (an SVD truncation, shaped like a LoRA) and a residual that
quantizes to 4 bits with less error; the low-rank part and any user LoRA run
in the same fused pass as the activation quantization.

Preparation is a one-time conversion of a checkpoint and runs on the host in
fp64 (numpy): the smoothing factors, the SVD and the residual.  The residual
is then quantized by the GPU library, and every per-call step of the layer
runs in the GPU kernels (nvfp4_gemm_w4a4_svdq).

Conventions (the pages leave them open):
  lambda_k = fp32(sqrt(a_k / w_k)), a_k = calibration max |x| of channel k,
             w_k = max_n |W[n, k]| (migration strength 1/2); 1 if either is 0
  smooth_k = fp32(1 / lambda_k): the kernel's input is bf16(x_k smooth_k)
  W'       = fp32(W diag(lambda))
  W' = U S V^T (fp64 SVD); up = bf16(U_r sqrt(S_r)) [N, r],
             down = bf16(sqrt(S_r) V_r^T) [r, K] (the split that balances the
             two factors' magnitudes for bf16)
  R        = fp32(W' - up down) with the bf16 factors, then NVFP4-quantized
"""
import numpy as np
import torch

from . import nvfp4 as nv


def smoothing(act_amax, w_amax):
    """(lambda, smooth) fp32 [K] from the per-channel activation and weight ranges."""
    a = np.asarray(act_amax, dtype=np.float32).astype(np.float64)
    w = np.asarray(w_amax, dtype=np.float32).astype(np.float64)
    if a.shape != w.shape or a.ndim != 1:
        raise ValueError("act_amax and w_amax must be [K] vectors")
    ok = (a != 0) & (w != 0)
    q = np.divide(a, w, out=np.ones_like(a), where=ok)
    lam = np.where(ok, np.sqrt(q), 1.0).astype(np.float32)
    smooth = (1.0 / lam.astype(np.float64)).astype(np.float32)
    return lam, smooth


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def factors(w, act_amax, rank, lora=None):
    """Host-side SVDQuant split of W [N, K] (fp32).

    Returns dict(lam, smooth [K] fp32, down [r', K] and up [N, r'] bf16 bit
    patterns, residual [N, K] fp32), r' = rank plus the rank of an optional
    user LoRA (A [rl, K], B [N, rl], fp32 values), appended as extra rows of
    down (A diag(lambda), since the layer's input is x / lambda) and columns
    of up."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if rank < 1 or rank > min(N, K):
        raise ValueError("rank must be in [1, min(N, K)]")
    lam, smooth = smoothing(act_amax, np.abs(w).max(axis=0))
    ws = (w.astype(np.float64) * lam.astype(np.float64)).astype(np.float32)
    u, s, vt = np.linalg.svd(ws.astype(np.float64), full_matrices=False)
    root = np.sqrt(s[:rank])
    up = _bf16_bits(u[:, :rank] * root)
    down = _bf16_bits(root[:, None] * vt[:rank])
    resid = (ws.astype(np.float64) - _bits_to_f64(up) @ _bits_to_f64(down)).astype(np.float32)
    if lora is not None:
        a_l, b_l = (np.asarray(t, dtype=np.float32) for t in lora)
        if a_l.ndim != 2 or a_l.shape[1] != K or b_l.shape != (N, a_l.shape[0]):
            raise ValueError("lora = (A [rl, K], B [N, rl])")
        down = np.concatenate([down, _bf16_bits(a_l.astype(np.float64) * lam.astype(np.float64))])
        up = np.concatenate([up, _bf16_bits(b_l)], axis=1)
    return {"lam": lam, "smooth": smooth, "down": down, "up": np.ascontiguousarray(up), "residual": resid}


def prepare(w, act_amax, rank, method="mse", lora=None, device="cuda"):
    """Device-ready SVDQuant layer: dict(smooth fp32 [K], down bf16 [r', K],
    up bf16 [N, r'], codes, scales, global) with the residual quantized on the
    GPU (method "mse", "absmax" or "4o6").  The total rank r' must be a
    multiple of 16 (at most 128), as the fused kernel requires."""
    f = factors(w, act_amax, rank, lora)
    r = f["down"].shape[0]
    if r % 16 != 0 or r > 128:
        raise ValueError("total low-rank size must be 16, 32, ..., 128")
    quant = {"mse": nv.quantize_mse, "absmax": nv.quantize_absmax, "4o6": nv.quantize_4o6}[method]
    codes, scales, glob = quant(torch.from_numpy(f["residual"]).to(device))

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)

    return {"smooth": torch.from_numpy(f["smooth"]).to(device), "down": bf16_dev(f["down"]),
            "up": bf16_dev(f["up"]), "codes": codes, "scales": scales, "global": glob, "lam": f["lam"]}


def forward(x, layer, out_dtype=torch.bfloat16, workspace=None, a_global=None):
    """y for bf16 x [M, K] through a prepared layer (one fused GPU call)."""
    return nv.gemm_w4a4(x, layer["codes"], layer["scales"], layer["global"], a_global=a_global,
                        out_dtype=out_dtype, workspace=workspace, lora=(layer["down"], layer["up"]),
                        smooth=layer["smooth"])
