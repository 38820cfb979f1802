"""Helpers for the GPU parity tests: move bf16 bit patterns to and from the
device, and compare the HIP results with the oracle."""
import sys

import numpy as np

BF16_O_TOL = 1.5e-2   # |O_gpu - O_oracle| for bf16 inputs
BF16_LSE_TOL = 1e-3   # |lse_gpu - lse_oracle| for bf16 inputs
F32_TOL = 2e-5        # |O_gpu - O_oracle| and lse for fp32 inputs


def say(*a):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def dev_f32(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_bf16_as_f64(t) -> np.ndarray:
    import torch
    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def host_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, want, tol):
    """Assert max |got - want| <= tol and print the measured error."""
    e = max_err(got, want)
    print(f"  {name}: max|err| = {e:.3e} (bar {tol:.1e})", flush=True)
    assert e <= tol, f"{name}: {e} > {tol}"


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0
