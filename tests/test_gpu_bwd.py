"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle's
attention_backward, through the C ABI.

Bar: every element of dq, dk and dv lies within the first-order error bound
of gpu_helpers.bwd_error_bounds, derived from fa_bwd's arithmetic (bf16
rounding of P, dS and the outputs, fp32 sums, and the O and lse the kernel is
given).  The kernel receives the oracle's O rounded to bf16 and its lse
rounded to fp32, except in the composed test, which feeds it fa_fwd's own
outputs.
"""
import numpy as np
import pytest

import oracle
from exact_tiled_attention_02_amd import inputs
from gpu_helpers import (bwd_error_bounds, check_bounded, dev_bf16, host_bf16_as_f64, host_f64,
                         say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_02_amd import fa
    fa.load()   # must load: no silent fallback


def to_bf16_bits(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, np.float64).astype(np.float32))


def run_bwd(q, k, v, o_bits, lse32, do, causal, scale):
    """fa_bwd on bf16 bit-pattern inputs; outputs start as NaN so that any
    element the kernels fail to write shows up."""
    from exact_tiled_attention_02_amd import fa
    B, Hq, Tq, d = q.shape
    _, Hkv, Tk, _ = k.shape
    tq, tk, tv, to, tdo = (dev_bf16(x) for x in (q, k, v, o_bits, do))
    tl = torch.from_numpy(np.ascontiguousarray(lse32, np.float32)).cuda()
    dq = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    dk = torch.full(k.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    dv = torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.fa_bwd(tq, tk, tv, to, tl, tdo, dq, dk, dv, B, Hq, Hkv, Tq, Tk, d, causal, scale,
              torch.cuda.current_stream())
    torch.cuda.synchronize()
    return host_bf16_as_f64(dq), host_bf16_as_f64(dk), host_bf16_as_f64(dv)


def parity(w: inputs.Prefill, scale=None, align="top_left"):
    causal = w.causal
    sc = w.scale if scale is None else scale
    q, k, v, do = inputs.prefill_inputs_with_grad(w)
    O, L = oracle.softmax_attention(q, k, v, causal=causal, scale=sc, align=align)
    o_bits = to_bf16_bits(O)
    lse32 = L.astype(np.float32)
    say("fa_bwd", w, align)
    mode = (2 if align == "bottom_right" else 1) if causal else 0
    dq, dk, dv = run_bwd(q, k, v, o_bits, lse32, do, mode, sc)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, causal=causal, scale=sc, align=align)
    bq, bk, bv = bwd_error_bounds(oracle.as_f64(q), oracle.as_f64(k), oracle.as_f64(v),
                                  oracle.as_f64(do), O, L, oracle.as_f64(o_bits),
                                  lse32.astype(np.float64), causal=causal, scale=sc,
                                  causal_off=oracle.causal_offset(w.Tq, w.Tk, align))
    check_bounded("dq", dq, rq, bq)
    check_bounded("dk", dk, rk, bk)
    check_bounded("dv", dv, rv, bv)
    return dq, dk, dv


SMALL = [
    # B, Hq, Hkv, Tq, Tk, d, causal
    (1, 1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (1, 2, 1, 7, 7, 64, True),
    (1, 1, 1, 13, 13, 128, False),
    (2, 4, 2, 100, 100, 64, True),
    (1, 8, 2, 257, 257, 128, True),
    (1, 4, 4, 130, 70, 64, False),     # Tq != Tk, non-causal
    (1, 4, 1, 65, 200, 128, True),     # Tq < Tk, causal: keys >= Tq get no gradient
    (1, 2, 2, 200, 65, 64, True),      # Tq > Tk, causal
    (2, 6, 3, 300, 300, 128, True),    # g = 2
    (1, 6, 2, 100, 100, 64, True),     # g = 3
    (1, 8, 1, 70, 70, 128, True),      # g = 8
    (1, 2, 1, 64, 64, 64, True),
    (1, 2, 2, 128, 128, 128, False),
    (1, 1, 1, 383, 383, 128, True),
    (1, 2, 1, 129, 385, 64, False),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_bwd_small_shapes(shape):
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    parity(inputs.Prefill("t", B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, causal=causal, seed=11))


BOTTOM_RIGHT = [
    # B, Hq, Hkv, Tq, Tk, d
    (1, 4, 2, 70, 300, 128),
    (1, 2, 1, 1, 257, 64),
    (2, 4, 4, 100, 100, 64),
    (1, 8, 2, 129, 1000, 64),
    (1, 2, 2, 200, 65, 128),     # Tq > Tk: the first 135 rows see no key
    (1, 6, 3, 33, 97, 128),
]


@pytest.mark.parametrize("shape", BOTTOM_RIGHT, ids=lambda s: "x".join(map(str, s)))
def test_bwd_bottom_right(shape):
    B, Hq, Hkv, Tq, Tk, d = shape
    dq, _, _ = parity(inputs.Prefill("t", B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, causal=True,
                                     seed=18), align="bottom_right")
    if Tq > Tk:
        assert np.all(dq[:, :, :Tq - Tk] == 0)


def test_bwd_keys_past_last_row_get_zero():
    """Causal with Tq < Tk: keys after the last query row are seen by no row."""
    w = inputs.Prefill("t", B=1, Hq=2, Hkv=1, Tq=40, Tk=300, d=64, causal=True, seed=12)
    _, dk, dv = parity(w)
    assert np.all(dk[:, :, 40:] == 0) and np.all(dv[:, :, 40:] == 0)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.3])
def test_bwd_other_scales(scale):
    parity(inputs.Prefill("t", B=1, Hq=2, Hkv=1, Tq=150, Tk=150, d=64, causal=True, seed=13),
           scale=scale)


def test_bwd_large_query_scale():
    """Q x 3 (the Qwen3-shaped workload's distribution): peaked rows."""
    parity(inputs.Prefill("t", B=1, Hq=4, Hkv=2, Tq=300, Tk=300, d=128, causal=True,
                          q_mult=3.0, seed=14))


def test_bwd_no_query_rows_zeroes_dk_dv():
    from exact_tiled_attention_02_amd import fa
    k = torch.randn(1, 2, 50, 64, device="cuda").to(torch.bfloat16)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(k, float("nan"))
    say("fa_bwd Tq=0")
    fa.fa_bwd(None, k, k, None, None, None, None, dk, dv, 1, 4, 2, 0, 50, 64, True, 0.125,
              torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.all(dk.float() == 0) and torch.all(dv.float() == 0)


def test_bwd_no_keys_zeroes_dq():
    from exact_tiled_attention_02_amd import fa
    q = torch.randn(1, 2, 70, 128, device="cuda").to(torch.bfloat16)
    lse = torch.full((1, 2, 70), float("-inf"), device="cuda")
    dq = torch.full_like(q, float("nan"))
    say("fa_bwd Tk=0")
    fa.fa_bwd(q, None, None, q, lse, q, dq, None, None, 1, 2, 2, 70, 0, 128, False, 0.1,
              torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.all(dq.float() == 0)


def test_bwd_empty_batch_is_noop():
    from exact_tiled_attention_02_amd import fa
    fa.fa_bwd(None, None, None, None, None, None, None, None, None, 0, 4, 2, 16, 16, 64, True,
              0.125)


def test_bwd_composed_with_fa_fwd():
    """fa_fwd's own O and lse feed fa_bwd (the training composition); the bound
    accounts for their measured deviation from the exact values."""
    from exact_tiled_attention_02_amd import fa
    w = inputs.Prefill("t", B=2, Hq=4, Hkv=2, Tq=333, Tk=333, d=128, causal=True, seed=15)
    q, k, v, do = inputs.prefill_inputs_with_grad(w)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.empty(tq.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(tq.shape[:3], dtype=torch.float32, device="cuda")
    say("fa_fwd + fa_bwd composed")
    fa.fa_fwd(tq, tk, tv, o, lse, 2, 4, 2, 333, 333, 128, True, w.scale,
              torch.cuda.current_stream())
    torch.cuda.synchronize()
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    lse32 = lse.cpu().numpy()
    dq, dk, dv = run_bwd(q, k, v, o_bits, lse32, do, True, w.scale)
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=w.scale)
    rq, rk, rv = oracle.attention_backward(q, k, v, do, causal=True, scale=w.scale)
    bq, bk, bv = bwd_error_bounds(oracle.as_f64(q), oracle.as_f64(k), oracle.as_f64(v),
                                  oracle.as_f64(do), O, L, oracle.as_f64(o_bits),
                                  lse32.astype(np.float64), causal=True, scale=w.scale)
    check_bounded("dq", dq, rq, bq)
    check_bounded("dk", dk, rk, bk)
    check_bounded("dv", dv, rv, bv)


def test_bwd_deterministic_and_inputs_untouched():
    from exact_tiled_attention_02_amd import fa
    w = inputs.Prefill("t", B=1, Hq=4, Hkv=1, Tq=515, Tk=515, d=128, causal=True, seed=16)
    q, k, v, do = inputs.prefill_inputs_with_grad(w)
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=w.scale)
    tens = [dev_bf16(x) for x in (q, k, v, to_bf16_bits(O), do)]
    tl = torch.from_numpy(L.astype(np.float32)).cuda()
    before = [t.clone() for t in tens] + [tl.clone()]
    outs = []
    say("fa_bwd determinism")
    for _ in range(2):
        g = [torch.empty_like(tens[0]), torch.empty_like(tens[1]), torch.empty_like(tens[2])]
        fa.fa_bwd(tens[0], tens[1], tens[2], tens[3], tl, tens[4], g[0], g[1], g[2],
                  1, 4, 1, 515, 515, 128, True, w.scale, torch.cuda.current_stream())
        torch.cuda.synchronize()
        outs.append([x.view(torch.int16).cpu() for x in g])
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    for a, b in zip(tens + [tl], before):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_bwd_qwen3_workload_two_groups_exact():
    """Full Qwen3-shaped launch (Hq=16, Hkv=8, T=4096, d=128, causal, Q x 3);
    the oracle checks every element of two kv-head groups (query heads 0, 1
    and 14, 15 with kv heads 0 and 7)."""
    from exact_tiled_attention_02_amd import fa
    w = inputs.QWEN3_0P6B_GQA
    q, k, v, do = inputs.prefill_inputs_with_grad(w)
    heads = [0, 1, 14, 15]
    kvh = [0, 7]
    qs, ks, vs, dos = q[:, heads], k[:, kvh], v[:, kvh], do[:, heads]
    O, L = oracle.softmax_attention(qs, ks, vs, causal=True, scale=w.scale)
    # Every head's O and lse for the launch: the sampled heads from the
    # oracle, the others from fa_fwd (their gradients are not checked).
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.empty(tq.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(tq.shape[:3], dtype=torch.float32, device="cuda")
    say("fa_fwd", w.name)
    fa.fa_fwd(tq, tk, tv, o, lse, w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, True, w.scale,
              torch.cuda.current_stream())
    torch.cuda.synchronize()
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    lse32 = lse.cpu().numpy().copy()
    o_bits[:, heads] = to_bf16_bits(O)
    lse32[:, heads] = L.astype(np.float32)
    say("fa_bwd", w.name)
    dq, dk, dv = run_bwd(q, k, v, o_bits, lse32, do, True, w.scale)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    rq, rk, rv = oracle.attention_backward(qs, ks, vs, dos, causal=True, scale=w.scale)
    bq, bk, bv = bwd_error_bounds(oracle.as_f64(qs), oracle.as_f64(ks), oracle.as_f64(vs),
                                  oracle.as_f64(dos), O, L, oracle.as_f64(o_bits[:, heads]),
                                  lse32[:, heads].astype(np.float64), causal=True, scale=w.scale)
    check_bounded("dq", dq[:, heads], rq, bq)
    check_bounded("dk", dk[:, kvh], rk, bk)
    check_bounded("dv", dv[:, kvh], rv, bv)


def test_bwd_llama3_long_workload_sampled():
    """Full Llama-3-shaped launch (Hq=32, Hkv=8, T=32768, d=128, causal) fed
    fa_fwd's O and lse.  The oracle checks, for query heads 20 and 21 of kv
    head 5: dq of the first 32, the last 32 and 32 random rows, each from that
    row alone (keys 0..i, no mask); and the two heads' contributions to dk and
    dv of the last 64 keys, which only the last 64 rows see, summed from those
    rows one by one, against the same heads' share computed on the GPU by a
    second launch restricted to them (Hq=2, Hkv=1).  The full launch's dk and
    dv of those keys must equal the sum of the four query heads' shares."""
    from exact_tiled_attention_02_amd import fa
    w = inputs.LLAMA3_8B_LONG
    T, d, sc = w.Tq, w.d, w.scale
    q, k, v, do = inputs.prefill_inputs_with_grad(w)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.empty(tq.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(tq.shape[:3], dtype=torch.float32, device="cuda")
    say("fa_fwd", w.name)
    fa.fa_fwd(tq, tk, tv, o, lse, w.B, w.Hq, w.Hkv, T, T, d, True, sc, torch.cuda.current_stream())
    torch.cuda.synchronize()
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    lse32 = lse.cpu().numpy()
    del tq, tk, tv, o, lse
    say("fa_bwd", w.name)
    dq, dk, dv = run_bwd(q, k, v, o_bits, lse32, do, True, sc)
    kh = 5
    rng = np.random.default_rng(321)
    rows = sorted(set(range(32)) | set(range(T - 32, T)) |
                  set(rng.choice(np.arange(32, T - 32), 32, replace=False).tolist()))
    K = oracle.as_f64(k[0, kh])
    V = oracle.as_f64(v[0, kh])
    nlast = 64
    lo = T - nlast
    last = set(range(lo, T))
    share_k = np.zeros((4, nlast, d))
    share_v = np.zeros((4, nlast, d))
    for hh in range(4):
        h = 4 * kh + hh
        # This query head's share of dk, dv of kv head 5, from a launch with
        # only that head (its O and lse are the full launch's).
        sel = slice(h, h + 1)
        gq_, gk_, gv_ = run_bwd(q[:, sel], k[:, kh:kh + 1], v[:, kh:kh + 1], o_bits[:, sel],
                                lse32[:, sel], do[:, sel], True, sc)
        share_k[hh] = gk_[0, 0, lo:]
        share_v[hh] = gv_[0, 0, lo:]
        assert np.array_equal(gq_[0, 0], dq[0, h]), "dq of a head must not depend on the others"
        if hh >= 2:
            continue
        acc_k = np.zeros((nlast, d))
        acc_v = np.zeros((nlast, d))
        bnd_k = np.zeros((nlast, d))
        bnd_v = np.zeros((nlast, d))
        for i in sorted(set(rows) | last):
            qi = q[0, h, i:i + 1][None, None]
            doi = do[0, h, i:i + 1][None, None]
            ki = k[0, kh, :i + 1][None, None]
            vi = v[0, kh, :i + 1][None, None]
            Oi, Li = oracle.softmax_attention(qi, ki, vi, causal=False, scale=sc)
            gq, gk, gv = oracle.attention_backward(qi, ki, vi, doi, causal=False, scale=sc)
            bq, bk, bv = bwd_error_bounds(
                oracle.as_f64(qi), K[None, None, :i + 1], V[None, None, :i + 1],
                oracle.as_f64(doi), Oi, Li, oracle.as_f64(o_bits[0, h, i:i + 1])[None, None],
                lse32[0, h, i:i + 1].astype(np.float64)[None, None], causal=False, scale=sc,
                safety=1.0)
            if i in rows:
                check_bounded(f"dq[h{h},row {i}]", dq[0, h, i], gq[0, 0, 0], 1.25 * bq[0, 0, 0])
            if i in last:
                acc_k[: i + 1 - lo] += gk[0, 0, lo:]
                acc_v[: i + 1 - lo] += gv[0, 0, lo:]
                bnd_k[: i + 1 - lo] += bk[0, 0, lo:]
                bnd_v[: i + 1 - lo] += bv[0, 0, lo:]
        check_bounded(f"dk[h{h} share, last keys]", share_k[hh], acc_k, 1.25 * bnd_k)
        check_bounded(f"dv[h{h} share, last keys]", share_v[hh], acc_v, 1.25 * bnd_v)
    # The group sum: the full launch adds the four shares (each rounded to
    # bf16 above, so compare within the rounding of five bf16 values).
    for name, full, share in (("dk", dk, share_k), ("dv", dv, share_v)):
        tot = share.sum(axis=0)
        err = np.abs(full[0, kh, lo:] - tot)
        bound = 2.0 ** -8 * (np.abs(full[0, kh, lo:]) + np.abs(share).sum(axis=0)) * 1.25 + 1e-6
        print(f"  {name} group sum: max err/bound = {np.max(err / bound):.3f}", flush=True)
        assert np.all(err <= bound)


def test_bwd_large_grid_sampled_group():
    """A grid large enough for the 8-wavefront dQ workgroups (B=2, Hq=32,
    Hkv=8, T=2048, d=64, causal); the oracle checks every element of the
    kv-head group 1 of sequence 1 (query heads 4..7)."""
    from exact_tiled_attention_02_amd import fa
    w = inputs.Prefill("t", B=2, Hq=32, Hkv=8, Tq=2048, Tk=2048, d=64, causal=True, seed=17)
    q, k, v, do = inputs.prefill_inputs_with_grad(w)
    b, kh, heads = 1, 1, [4, 5, 6, 7]
    qs, ks, vs, dos = (q[b:b + 1, heads], k[b:b + 1, kh:kh + 1], v[b:b + 1, kh:kh + 1],
                       do[b:b + 1, heads])
    O, L = oracle.softmax_attention(qs, ks, vs, causal=True, scale=w.scale)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.empty(tq.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(tq.shape[:3], dtype=torch.float32, device="cuda")
    say("fa_fwd large grid")
    fa.fa_fwd(tq, tk, tv, o, lse, w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, True, w.scale,
              torch.cuda.current_stream())
    torch.cuda.synchronize()
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    lse32 = lse.cpu().numpy().copy()
    o_bits[b:b + 1, heads] = to_bf16_bits(O)
    lse32[b:b + 1, heads] = L.astype(np.float32)
    say("fa_bwd large grid")
    dq, dk, dv = run_bwd(q, k, v, o_bits, lse32, do, True, w.scale)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    rq, rk, rv = oracle.attention_backward(qs, ks, vs, dos, causal=True, scale=w.scale)
    bq, bk, bv = bwd_error_bounds(oracle.as_f64(qs), oracle.as_f64(ks), oracle.as_f64(vs),
                                  oracle.as_f64(dos), O, L, oracle.as_f64(o_bits[b:b + 1, heads]),
                                  lse32[b:b + 1, heads].astype(np.float64), causal=True,
                                  scale=w.scale)
    check_bounded("dq", dq[b:b + 1, heads], rq, bq)
    check_bounded("dk", dk[b:b + 1, kh:kh + 1], rk, bk)
    check_bounded("dv", dv[b:b + 1, kh:kh + 1], rv, bv)
