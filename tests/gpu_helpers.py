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


# ---------------------------------------------------------------------------
# Backward pass: element-wise error bounds
# ---------------------------------------------------------------------------
BF16_U = 2.0 ** -8    # unit roundoff of bf16 (8 significant bits, nearest even)
F32_U = 2.0 ** -24


def bwd_error_bounds(q, k, v, do, O, L, o_used, lse_used, *, causal, scale, safety=1.25,
                     causal_off=0):
    """First-order bounds on |kernel - exact| for dq, dk, dv, element by element.

    Inputs are fp64 [B,H,T,d] arrays: q, k, v, do as the kernel received them
    (bf16 values), O and L the exact forward output and row log-sum-exp, and
    o_used / lse_used the O and lse the kernel was given.  The arithmetic
    being bounded (fa_bwd's): P = exp(scale*q.k - lse_used) in fp32, rounded
    to bf16 for dV = P^T dO; D = dO . o_used in fp32; dS = P (dP - D) in fp32,
    rounded to bf16 for dQ = scale dS K and dK = scale dS^T Q; products exact
    in fp32, sums in fp32 over at most n terms; outputs rounded to bf16.
    Per visible (i, j), with u = 2^-8 and g = u + n 2^-24:
        rho_i   = expm1(|lse_used_i - L_i|) + 2^-21 (max_j |s_ij| + |L_i| + 1)
        dD_i    = sum_d |do_id| |o_used - O|_id + 2^-20 sum_d |do_id O_id|
        e_dS_ij = g |dS_ij| + rho_i P_ij |dP_ij - D_i| + P_ij dD_i
        |e dV_j| <= u |dV_j| + sum_i (g + rho_i) P_ij |do_i|
        |e dQ_i| <= u |dQ_i| + |scale| sum_j e_dS_ij |k_j|
        |e dK_j| <= u |dK_j| + |scale| sum_i e_dS_ij |q_i|
    times `safety`, plus 1e-6 * max(1, max|ref|) per tensor.  Returns
    (bdq, bdk, bdv)."""
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    n = max(Tq, Tk, 1)
    gam = BF16_U + n * F32_U
    bdq = np.zeros(q.shape)
    bdk = np.zeros(k.shape)
    bdv = np.zeros(v.shape)
    rdq = np.zeros(q.shape)
    rdk = np.zeros(k.shape)
    rdv = np.zeros(v.shape)
    if Tq == 0 or Tk == 0:
        return bdq, bdk, bdv
    i_idx = np.arange(Tq)[:, None]
    j_idx = np.arange(Tk)[None, :]
    vis = (j_idx <= i_idx + causal_off) if causal else np.ones((Tq, Tk), bool)
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            s = scale * (q[b, h] @ k[b, kh].T)
            Lf = np.where(np.isfinite(L[b, h]), L[b, h], 0.0)
            P = np.where(vis, np.exp(np.where(vis, s, 0.0) - Lf[:, None]), 0.0)
            dP = do[b, h] @ v[b, kh].T
            D = np.sum(do[b, h] * O[b, h], axis=1)
            dS = P * (dP - D[:, None])
            smax = np.max(np.where(vis, np.abs(s), 0.0), axis=1)
            has = np.isfinite(L[b, h])   # rows with no visible key have P = 0
            dlse = np.where(has, np.abs(np.where(has, lse_used[b, h], 0) - np.where(has, L[b, h], 0)), 0)
            rho = np.expm1(dlse) + 2.0 ** -21 * (smax + np.where(has, np.abs(L[b, h]), 0) + 1)
            dD = (np.sum(np.abs(do[b, h]) * np.abs(o_used[b, h] - O[b, h]), axis=1) +
                  2.0 ** -20 * np.sum(np.abs(do[b, h] * O[b, h]), axis=1))
            edS = gam * np.abs(dS) + rho[:, None] * P * np.abs(dP - D[:, None]) + P * dD[:, None]
            bdv[b, kh] += P.T @ ((gam + rho)[:, None] * np.abs(do[b, h]))
            bdq[b, h] = abs(scale) * (edS @ np.abs(k[b, kh]))
            bdk[b, kh] += abs(scale) * (edS.T @ np.abs(q[b, h]))
            rdq[b, h] = scale * (dS @ k[b, kh])
            rdk[b, kh] += scale * (dS.T @ q[b, h])
            rdv[b, kh] += P.T @ do[b, h]
    out = []
    for bnd, ref in ((bdq, rdq), (bdk, rdk), (bdv, rdv)):
        floor = 1e-6 * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
        out.append(safety * (bnd + BF16_U * np.abs(ref)) + floor)
    return tuple(out)


def check_bounded(name, got, want, bound):
    """Assert |got - want| <= bound element-wise; print the worst ratio."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if got.size == 0:
        print(f"  {name}: empty", flush=True)
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - want)
    ratio = float(np.max(err / bound))
    print(f"  {name}: max|err| = {np.max(err):.3e}, max|ref| = {np.max(np.abs(want)):.3e}, "
          f"max err/bound = {ratio:.3f}", flush=True)
    assert ratio <= 1.0, f"{name}: error exceeds its bound (ratio {ratio:.3f})"


# ---------------------------------------------------------------------------
# 8-bit forward: element-wise error bound
# ---------------------------------------------------------------------------
E4M3_U = 2.0 ** -4            # relative rounding of an E4M3 normal value (3 mantissa bits)
E4M3_FLOOR = 2.0 ** -10 / 448  # absolute rounding of 448 * P below the smallest normal, in P units


def fp8_fwd_error_bound(q, k, v, *, causal, scale, causal_off=0, safety=1.25):
    """Bound on |O_kernel - O_exact| for fa_fwd_fp8, element by element.

    q, k, v: the dequantised fp64 inputs.  The only rounding of consequence
    is that of each probability P_ij = exp(s_ij - m_i) <= 1 (times 448) to
    E4M3 before the P.V product: |dP| <= max(2^-4 P, 2^-10/448).  With the
    row sum l_i = sum_j P_ij unrounded,
        |O_err[i, c]| <= sum_j max(2^-4 P_ij, 2^-10/448) |v_jc| / l_i,
    plus the bf16 rounding of O (2^-8 |O|); times `safety`, plus 1e-6."""
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    bound = np.zeros((B, Hq, Tq, v.shape[3]))
    O = np.zeros_like(bound)
    i_idx = np.arange(Tq)[:, None]
    j_idx = np.arange(Tk)[None, :]
    vis = (j_idx <= i_idx + causal_off) if causal else np.ones((Tq, Tk), bool)
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            s = np.where(vis, scale * (q[b, h] @ k[b, kh].T), -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            P = np.where(vis, np.exp(s - m), 0.0)
            l = P.sum(axis=1, keepdims=True)
            lsafe = np.where(l > 0, l, 1.0)
            dP = np.where(vis, np.maximum(E4M3_U * P, E4M3_FLOOR), 0.0)
            bound[b, h] = (dP @ np.abs(v[b, kh])) / lsafe
            O[b, h] = (P @ v[b, kh]) / lsafe
    return safety * (bound + 2.0 ** -8 * np.abs(O)) + 1e-6
