"""Shared helpers for the GPU parity tests (device transfers, bracket checks)."""
import numpy as np
import torch

import oracle

DEV = "cuda:0"


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bracket_bf16(y_bits, ystar, tau, what=""):
    """GPU bf16 outputs must lie in [bf16(y* - tau), bf16(y* + tau)]."""
    y = bf16_bits_to_f64(y_bits)
    lo, hi = oracle.bracket_bf16(ystar, tau)
    bad = ~((lo <= y) & (y <= hi))
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outputs outside the bracket; first "
                             f"{list(zip(y[i], ystar[i], tau[i]))}")


def assert_within_tau(y32, ystar, tau, what=""):
    err = np.abs(np.asarray(y32, dtype=np.float64) - ystar)
    bad = err > tau
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outputs beyond tau; first "
                             f"{list(zip(err[i], tau[i]))}")
    return float((err / np.maximum(tau / 1e-5, 1e-300)).max())
