"""Helpers for the GPU parity tests: move bf16 bit patterns to and from the
device, and compare the HIP results with the oracle."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

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


def pool_workers() -> int:
    """Threads for oracle work: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def head_map(fn, items):
    """fn over items on a thread pool, one-threaded BLAS inside each call (the
    oracle's array operations release the interpreter lock)."""
    from threadpoolctl import threadpool_limits
    items = list(items)
    with threadpool_limits(1):
        with ThreadPoolExecutor(pool_workers()) as ex:
            return list(ex.map(fn, items))


def check_every_element(O, L, q, k, v, *, causal, scale, align="top_left",
                        o_tol=None, lse_tol=None):
    """Compare every element of O [B,Hq,Tq,d] and L [B,Hq,Tq] with the oracle,
    one (batch, head) per task.  Returns (max |O err|, max |lse err|)."""
    import oracle
    o_tol = BF16_O_TOL if o_tol is None else o_tol
    lse_tol = BF16_LSE_TOL if lse_tol is None else lse_tol
    B, Hq = q.shape[:2]
    g = Hq // k.shape[1]

    def one(bh):
        b, h = bh
        kv = h // g
        Or, Lr = oracle.softmax_attention(q[b:b + 1, h:h + 1], k[b:b + 1, kv:kv + 1],
                                          v[b:b + 1, kv:kv + 1], causal=causal, scale=scale,
                                          align=align)
        return max_err(O[b, h], Or[0, 0]), max_err(L[b, h], Lr[0, 0])

    errs = head_map(one, [(b, h) for b in range(B) for h in range(Hq)])
    eo = max(e[0] for e in errs) if errs else 0.0
    el = max(e[1] for e in errs) if errs else 0.0
    print(f"  O: max|err| = {eo:.3e} (bar {o_tol:.1e}) over {B * Hq} heads", flush=True)
    print(f"  lse: max|err| = {el:.3e} (bar {lse_tol:.1e})", flush=True)
    assert eo <= o_tol, f"O: {eo} > {o_tol}"
    assert el <= lse_tol, f"lse: {el} > {lse_tol}"
    return eo, el


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
# Decode: element-wise error bound
# ---------------------------------------------------------------------------
def decode_error_bound(q, K, V, seqlens, *, safety=1.25):
    """Bound on |O_kernel - O_exact| for fa_decode (bf16 cache) and
    fa_decode_fp8 / fa_decode_int8 (8-bit codes with per-row scales), element
    by element.

    q: [B, Hq, d] fp64 queries; K, V: [B, Hkv, Tmax, d] fp64 cache rows as
    the oracle reads them (dequantised; only each sequence's valid prefix is
    used).  The kernels form scores from exact bf16 products with fp32 sums,
    P_j = 2^(s_j c - m c) in fp32, the row sum l from the unrounded P, and
    round P_j (times the V row scale, for 8-bit caches) to bf16 before the
    P.V product, which sums in fp32; partial results merge by the rescale
    rule in fp32 and O is rounded to bf16.  So, with A = sum_j P_j |v_j| / l:
      * rounding P to bf16: at most 2^-8 A;
      * rounding O to bf16: at most 2^-8 |O|;
      * the fp32 score and exponent error, a relative error ds of every P_j:
        at most ds (A + |O|), ds = (d + 4) 2^-24 |scale| max_j sum_i |q_i k_ji|
        + 2^-21;
    plus the fp32 sums (n 2^-24 relative, absorbed by `safety`) and 1e-6."""
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(d)
    out = np.full((B, Hq, V.shape[3]), 1e-6)
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        for h in range(Hq):
            k = K[b, h // g, :n]
            v = V[b, h // g, :n]
            s = scale * (k @ q[b, h])
            P = np.exp(s - s.max())
            l = P.sum()
            A = (P @ np.abs(v)) / l
            O = (P @ v) / l
            ds = (d + 4) * 2.0 ** -24 * scale * float(np.max(np.abs(k) @ np.abs(q[b, h]))) + 2.0 ** -21
            out[b, h] = safety * (2.0 ** -8 + ds) * (A + np.abs(O)) + 1e-6
    return out


# ---------------------------------------------------------------------------
# 8-bit forward: element-wise error bound
# ---------------------------------------------------------------------------
E4M3_U = 2.0 ** -4            # relative rounding of an E4M3 normal value (3 mantissa bits)
F8_HEADROOM = 1                # bits between a tile's largest probability and the largest E4M3 code
# Absolute rounding of a probability code below the smallest normal, in P
# units: the kernel codes each tile's probabilities with a power-of-two
# factor that puts the tile's largest between 448 * 2^-F8_HEADROOM and 448,
# i.e. a factor of at least 448 * 2^-F8_HEADROOM per unit of P (no tile's
# max exceeds the row's), and a subnormal code rounds by at most 2^-10.
E4M3_FLOOR = 2.0 ** (F8_HEADROOM - 10) / 448


def fp8_fwd_error_bound(q, k, v, *, causal, scale, causal_off=0, safety=1.25):
    """Bound on |O_kernel - O_exact| for fa_fwd_fp8, element by element.

    q, k, v: the dequantised fp64 inputs.  The only rounding of consequence
    is that of each probability P_ij = exp(s_ij - m_i) <= 1 (coded with a
    per-tile power-of-two factor of at least 448 * 2^-F8_HEADROOM) to E4M3
    before the P.V product: |dP| <= max(2^-4 P, E4M3_FLOOR).  With the row sum
    l_i = sum_j P_ij unrounded,
        |O_err[i, c]| <= sum_j max(2^-4 P_ij, E4M3_FLOOR) |v_jc| / l_i,
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


def fp8_fwd_error_bound_rows(q, k, v, rows, *, causal, scale, causal_off=0, safety=1.25):
    """fp8_fwd_error_bound for selected query rows of one head: q [n, d] the
    dequantised rows, rows [n] their positions, k, v [Tk, d] the dequantised
    keys and values of the head's kv head."""
    rows = np.asarray(rows)
    Tk = k.shape[0]
    vis = (np.arange(Tk)[None, :] <= rows[:, None] + causal_off) if causal else \
        np.ones((len(rows), Tk), bool)
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    P = np.where(vis, np.exp(s - m), 0.0)
    l = P.sum(axis=1, keepdims=True)
    lsafe = np.where(l > 0, l, 1.0)
    dP = np.where(vis, np.maximum(E4M3_U * P, E4M3_FLOOR), 0.0)
    bound = (dP @ np.abs(v)) / lsafe
    O = (P @ v) / lsafe
    return safety * (bound + 2.0 ** -8 * np.abs(O)) + 1e-6


def check_fp8_every_head(O, L, q8, k8, v8, qs, ks, vs, *, causal, scale, align="top_left",
                         heads=None):
    """Every element of the listed (batch, query head) pairs of an 8-bit
    forward (all pairs by default) against the oracle on the dequantised
    inputs: O within fp8_fwd_error_bound, lse within BF16_LSE_TOL.  One pair
    per thread-pool task.  Returns (worst err/bound, max |lse err|)."""
    import oracle
    B, Hq, Tq = q8.shape[:3]
    Tk = k8.shape[2]
    g = Hq // k8.shape[1]
    off = oracle.causal_offset(Tq, Tk, align)
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)

    def one(bh):
        b, h = bh
        kv = h // g
        sq, skv = (slice(b, b + 1), slice(h, h + 1)), (slice(b, b + 1), slice(kv, kv + 1))
        q, k, v = oracle.fp8_attention_inputs(q8[sq], k8[skv], v8[skv], qs[sq], ks[skv], vs[skv])
        Or, Lr = oracle.softmax_attention(q, k, v, causal=causal, scale=scale, align=align)
        bound = fp8_fwd_error_bound(q, k, v, causal=causal, scale=scale, causal_off=off)
        got = O[sq]
        ok = bool(np.all(np.isfinite(got)))
        ratio = float(np.max(np.abs(got - Or) / bound)) if got.size else 0.0
        return ok, ratio, max_err(L[sq], Lr)

    res = head_map(one, heads)
    finite = all(r[0] for r in res)
    ratio = max((r[1] for r in res), default=0.0)
    el = max((r[2] for r in res), default=0.0)
    print(f"  O: max err/bound = {ratio:.3f} over {len(heads)} heads", flush=True)
    print(f"  lse: max|err| = {el:.3e} (bar {BF16_LSE_TOL:.1e})", flush=True)
    assert finite, "non-finite output"
    assert ratio <= 1.0, f"O error exceeds its bound (ratio {ratio:.3f})"
    assert el <= BF16_LSE_TOL, f"lse: {el} > {BF16_LSE_TOL}"
    return ratio, el


def lse_error_bound(q, k, L, *, causal, scale, causal_off=0, safety=1.25):
    """Bound on |lse_kernel - lse_exact| per query row for bf16 inputs.

    q, k: fp64 values of the bf16 inputs [B,Hq,Tq,d], [B,Hkv,Tk,d]; L the
    exact lse.  A product of two bf16 values is exact in fp32 and the kernel
    sums the d products of a score in fp32, so each computed score is off
    by at most g_d sum_t |q_it k_jt| (g_d = d 2^-24 / (1 - d 2^-24)); the
    log-sum-exp moves by at most |scale| times the largest score error.  The
    rest is fp32 rounding of O(1) relative size: of c = |scale| log2(e), of
    the exponent arguments, of the n-term row sum, of log2 and of the final
    conversion to a natural log, together at most
    (8 |L_i| + n + 16) 2^-24.  Times `safety`.  Rows with no visible key
    (L = -inf) get 0."""
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    gd = d * F32_U / (1 - d * F32_U)
    n = max(Tk, 1)
    out = np.zeros((B, Hq, Tq))
    i_idx = np.arange(Tq)[:, None]
    j_idx = np.arange(Tk)[None, :]
    vis = (j_idx <= i_idx + causal_off) if causal else np.ones((Tq, Tk), bool)
    for b in range(B):
        for h in range(Hq):
            mag = np.abs(q[b, h]) @ np.abs(k[b, h // g]).T
            worst = np.max(np.where(vis, mag, 0.0), axis=1) if Tk else np.zeros(Tq)
            Lf = np.where(np.isfinite(L[b, h]), np.abs(L[b, h]), 0.0)
            e = abs(scale) * gd * worst + (8 * Lf + n + 16) * F32_U
            out[b, h] = np.where(np.isfinite(L[b, h]), safety * e, 0.0)
    return out
