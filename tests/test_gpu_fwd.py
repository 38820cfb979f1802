"""GPU parity of the forward kernels (fa_fwd bf16, fa_fwd_f32) against the
fp64 CPU oracle, through the C ABI.

Bars: bf16 inputs |O err| <= 1.5e-2 and |lse err| <= 1e-3; fp32 inputs
<= 2e-5 for both.
"""
import math

import numpy as np
import pytest

import oracle
from exact_tiled_attention_02_amd import inputs
from gpu_helpers import (BF16_LSE_TOL, BF16_O_TOL, F32_TOL, check, dev_bf16, dev_f32,
                         host_bf16_as_f64, host_f64, max_err, say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_02_amd import fa
    fa.load()   # must load: no silent fallback


def run_bf16(q, k, v, causal, scale, with_lse=True):
    from exact_tiled_attention_02_amd import fa
    B, Hq, Tq, d = q.shape
    _, Hkv, Tk, _ = k.shape
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.full((B, Hq, Tq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    fa.fa_fwd(tq, tk, tv, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale,
              torch.cuda.current_stream())
    torch.cuda.synchronize()
    return host_bf16_as_f64(o), (host_f64(lse) if with_lse else None)


def run_f32(q, k, v, causal, scale):
    from exact_tiled_attention_02_amd import fa
    B, Hq, Tq, d = q.shape
    _, Hkv, Tk, _ = k.shape
    tq, tk, tv = dev_f32(q), dev_f32(k), dev_f32(v)
    o = torch.full((B, Hq, Tq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_f32(tq, tk, tv, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale,
                  torch.cuda.current_stream())
    torch.cuda.synchronize()
    return host_f64(o), host_f64(lse)


SMALL = [
    # B, Hq, Hkv, Tq, Tk, d, causal
    (1, 1, 1, 1, 1, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (1, 2, 1, 7, 7, 64, True),
    (1, 1, 1, 13, 13, 128, False),
    (2, 4, 2, 100, 100, 64, True),
    (1, 8, 2, 257, 257, 128, True),
    (1, 4, 4, 130, 70, 64, False),     # Tq != Tk, non-causal
    (1, 4, 1, 65, 200, 128, True),     # Tq < Tk, causal (top-left)
    (1, 2, 2, 200, 65, 64, True),      # Tq > Tk, causal
    (2, 6, 3, 300, 300, 128, True),    # g = 2
    (1, 6, 2, 100, 100, 64, True),     # g = 3
    (1, 8, 1, 70, 70, 128, True),      # g = 8
    (1, 2, 1, 64, 64, 64, True),
    (1, 2, 2, 128, 128, 128, False),
    (1, 1, 1, 383, 383, 128, True),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_bf16_small_shapes(shape):
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    w = inputs.Prefill("t", B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, causal=causal, seed=7)
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd bf16", shape)
    O, L = run_bf16(q, k, v, causal, w.scale)
    Or, Lr = oracle.softmax_attention(q, k, v, causal=causal, scale=w.scale)
    check("O", O, Or, BF16_O_TOL)
    check("lse", L, Lr, BF16_LSE_TOL)


@pytest.mark.parametrize("shape", SMALL[:10], ids=lambda s: "x".join(map(str, s)))
def test_f32_small_shapes(shape):
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    w = inputs.Prefill("t", B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, causal=causal, dtype="f32",
                       seed=8)
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd_f32", shape)
    O, L = run_f32(q, k, v, causal, w.scale)
    Or, Lr = oracle.softmax_attention(q, k, v, causal=causal, scale=w.scale)
    check("O", O, Or, F32_TOL)
    check("lse", L, Lr, F32_TOL)


BOTTOM_RIGHT = [
    # B, Hq, Hkv, Tq, Tk, d
    (1, 4, 2, 70, 300, 128),
    (1, 2, 1, 1, 257, 64),
    (2, 4, 4, 100, 100, 64),
    (1, 8, 2, 129, 1000, 64),
    (1, 2, 2, 200, 65, 128),     # Tq > Tk: the first 135 rows see no key
    (1, 6, 3, 33, 97, 128),
    (1, 16, 4, 700, 2100, 128),  # a grid small enough for paired half-tiles
]


@pytest.mark.parametrize("shape", BOTTOM_RIGHT, ids=lambda s: "x".join(map(str, s)))
def test_bf16_bottom_right(shape):
    from exact_tiled_attention_02_amd import fa
    B, Hq, Hkv, Tq, Tk, d = shape
    w = inputs.Prefill("t", B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, causal=True, seed=19)
    q, k, v = inputs.prefill_inputs(w)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.full((B, Hq, Tq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device="cuda")
    say("fa_fwd bf16 bottom-right", shape)
    fa.fa_fwd(tq, tk, tv, o, lse, B, Hq, Hkv, Tq, Tk, d, 2, w.scale, torch.cuda.current_stream())
    torch.cuda.synchronize()
    O, L = host_bf16_as_f64(o), host_f64(lse)
    Or, Lr = oracle.softmax_attention(q, k, v, causal=True, scale=w.scale, align="bottom_right")
    check("O", O, Or, BF16_O_TOL)
    check("lse", L, Lr, BF16_LSE_TOL)


@pytest.mark.parametrize("shape", BOTTOM_RIGHT[:6], ids=lambda s: "x".join(map(str, s)))
def test_f32_bottom_right(shape):
    from exact_tiled_attention_02_amd import fa
    B, Hq, Hkv, Tq, Tk, d = shape
    w = inputs.Prefill("t", B=B, Hq=Hq, Hkv=Hkv, Tq=Tq, Tk=Tk, d=d, causal=True, dtype="f32",
                       seed=20)
    q, k, v = inputs.prefill_inputs(w)
    tq, tk, tv = dev_f32(q), dev_f32(k), dev_f32(v)
    o = torch.full((B, Hq, Tq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device="cuda")
    say("fa_fwd_f32 bottom-right", shape)
    fa.fa_fwd_f32(tq, tk, tv, o, lse, B, Hq, Hkv, Tq, Tk, d, 2, w.scale,
                  torch.cuda.current_stream())
    torch.cuda.synchronize()
    Or, Lr = oracle.softmax_attention(q, k, v, causal=True, scale=w.scale, align="bottom_right")
    check("O", host_f64(o), Or, F32_TOL)
    check("lse", host_f64(lse), Lr, F32_TOL)


def test_bottom_right_chunk_of_llama3_long_sampled():
    """Chunked prefill at full size: the last 4096 positions of a 32768-token
    Llama-3-shaped sequence (Hq=32, Hkv=8, d=128) against all 32768 cached
    keys; sampled rows of a spread of heads checked one by one."""
    from exact_tiled_attention_02_amd import fa
    w = inputs.Prefill("t", B=1, Hq=32, Hkv=8, Tq=4096, Tk=32768, d=128, causal=True, seed=21)
    q, k, v = inputs.prefill_inputs(w)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.empty((1, 32, 4096, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 32, 4096), dtype=torch.float32, device="cuda")
    say("fa_fwd bf16 bottom-right chunk 4096 of 32768")
    fa.fa_fwd(tq, tk, tv, o, lse, 1, 32, 8, 4096, 32768, 128, 2, w.scale,
              torch.cuda.current_stream())
    torch.cuda.synchronize()
    O, L = host_bf16_as_f64(o), host_f64(lse)
    rng = np.random.default_rng(5)
    for h in (0, 13, 31):
        rows = _sample_rows(4096, rng, n_random=64)
        Or, Lr = oracle.softmax_attention_rows(q, k, v, causal=True, scale=w.scale, b=0, h=h,
                                               rows=rows, align="bottom_right")
        check("O", O[0, h, rows], Or, BF16_O_TOL)
        check("lse", L[0, h, rows], Lr, BF16_LSE_TOL)


def test_single_head_f32_workload():
    """B=1, H=1, T=256, d=64, fp32, non-causal, seed 0."""
    w = inputs.SINGLE_HEAD_F32
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd_f32", w.name)
    O, L = run_f32(q, k, v, w.causal, w.scale)
    Or, Lr = oracle.softmax_attention(q, k, v, causal=w.causal, scale=w.scale)
    check("O", O, Or, F32_TOL)
    check("lse", L, Lr, F32_TOL)


def test_qwen3_gqa_workload_full():
    """Hq=16, Hkv=8, T=4096, d=128, causal, Q x 3: every output element."""
    w = inputs.QWEN3_0P6B_GQA
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd bf16", w.name)
    O, L = run_bf16(q, k, v, w.causal, w.scale)
    Or, Lr = oracle.softmax_attention(q, k, v, causal=w.causal, scale=w.scale)
    check("O", O, Or, BF16_O_TOL)
    check("lse", L, Lr, BF16_LSE_TOL)


def _sample_rows(T, rng, n_random=192):
    rows = set(range(0, min(T, 128))) | set(range(max(0, T - 128), T))
    rows |= set(rng.choice(T, size=min(T, n_random), replace=False).tolist())
    return sorted(rows)


@pytest.mark.parametrize("name", ["gpt2_small_mha", "llama3_8b_long"])
def test_full_size_workloads_sampled_rows(name):
    """Full-size launch; the oracle checks the first and last 128 rows and
    192 random rows of a spread of (batch, head) pairs one by one."""
    w = inputs.WORKLOADS[name]
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd bf16", w.name)
    O, L = run_bf16(q, k, v, w.causal, w.scale)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    rng = np.random.default_rng(123)
    pairs = [(0, 0), (w.B - 1, w.Hq - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.Hq)))
                                             for _ in range(4)]
    for b, h in pairs:
        rows = _sample_rows(w.Tq, rng)
        Or, Lr = oracle.softmax_attention_rows(q, k, v, causal=w.causal, scale=w.scale, b=b, h=h,
                                               rows=rows)
        check("O", O[b, h, rows], Or, BF16_O_TOL)
        check("lse", L[b, h, rows], Lr, BF16_LSE_TOL)


@pytest.mark.parametrize("shape", [
    (1, 32, 8, 4096, 128, 3.0),   # 512 paired workgroups: light/heavy wavefront pairs
    (1, 12, 12, 4096, 64, 1.0),   # 384 paired workgroups, d = 64: key split
    (1, 16, 8, 2048, 128, 1.0),   # 128 paired workgroups: key split, GQA
], ids=lambda s: "x".join(map(str, s)))
def test_small_causal_grids_sampled_rows(shape):
    """Causal grids under four workgroups per compute unit balance the
    triangle by pairing light and heavy half-tiles, either with the key split
    or with light/heavy wavefront pairs, depending on the grid size.  Both
    schemes are checked on sampled rows of every head."""
    B, Hq, Hkv, T, d, qm = shape
    w = inputs.Prefill("t", B=B, Hq=Hq, Hkv=Hkv, Tq=T, Tk=T, d=d, causal=True, q_mult=qm, seed=21)
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd bf16 small causal grid", shape)
    O, L = run_bf16(q, k, v, True, w.scale)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    rng = np.random.default_rng(7)
    for h in range(Hq):
        rows = sorted(set(rng.choice(T, size=24, replace=False).tolist()) | {0, 31, 32, T // 2, T - 1})
        Or, Lr = oracle.softmax_attention_rows(q, k, v, causal=True, scale=w.scale, b=0, h=h, rows=rows)
        check("O", O[0, h, rows], Or, BF16_O_TOL)
        check("lse", L[0, h, rows], Lr, BF16_LSE_TOL)


def test_large_query_scale_stability():
    """Q x 100 ([FUSED07] task 07.2, requirement 4): finite, matches the oracle."""
    w = inputs.Prefill("t", B=1, Hq=4, Hkv=2, Tq=300, Tk=300, d=128, causal=True, q_mult=100.0,
                       seed=3)
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd bf16 Qx100")
    O, L = run_bf16(q, k, v, True, w.scale)
    Or, Lr = oracle.softmax_attention(q, k, v, causal=True, scale=w.scale)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    check("O", O, Or, BF16_O_TOL)
    # lse ~ 1e3 here; the bar is relative to fp32 rounding of such values.
    check("lse", L, Lr, max(BF16_LSE_TOL, 4e-6 * np.max(np.abs(Lr))))


@pytest.mark.parametrize("d,growth", [(64, 3.0), (128, 3.0), (128, 12.0), (64, 0.4)])
def test_slowly_growing_row_max(d, growth):
    """Scores that rise along the key sequence, so every row's max grows tile
    after tile by about `growth` powers of 2 per 64 keys.  The kernel moves
    its reference max only when a row has outgrown it by more than 2^8, so
    here most tiles run against a stale reference with probabilities above 1
    (growth 3 and 0.4), or every tile moves it (growth 12); rows are peaked
    on their last keys.  Output and lse must still match the oracle."""
    rng = np.random.default_rng(11)
    Tq = Tk = 1000
    scale = 1.0 / math.sqrt(d)
    c = scale * math.log2(math.e)
    slope = growth / (64.0 * c)          # raw score increase per key
    q = 0.5 * rng.standard_normal((1, 2, Tq, d)).astype(np.float32)
    q[..., 0] += 1.0
    k = rng.standard_normal((1, 1, Tk, d)).astype(np.float32)
    k[..., 0] += slope * np.arange(Tk, dtype=np.float32)
    v = rng.standard_normal((1, 1, Tk, d)).astype(np.float32)
    q, k, v = (inputs.f32_to_bf16_bits(x) for x in (q, k, v))
    say("fa_fwd bf16 rising scores d", d, "growth", growth)
    O, L = run_bf16(q, k, v, True, scale)
    Or, Lr = oracle.softmax_attention(q, k, v, causal=True, scale=scale)
    check("O", O, Or, BF16_O_TOL)
    check("lse", L, Lr, BF16_LSE_TOL)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5])
def test_other_scales(scale):
    w = inputs.Prefill("t", B=1, Hq=2, Hkv=1, Tq=150, Tk=150, d=64, causal=True, seed=4)
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd bf16 scale", scale)
    O, L = run_bf16(q, k, v, True, scale)
    Or, Lr = oracle.softmax_attention(q, k, v, causal=True, scale=scale)
    check("O", O, Or, BF16_O_TOL)
    check("lse", L, Lr, BF16_LSE_TOL)


def test_no_keys_gives_zero_and_minus_inf():
    from exact_tiled_attention_02_amd import fa
    q = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    o = torch.full((1, 2, 5, 64), float("nan"), device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 5, device="cuda")
    say("fa_fwd bf16 Tk=0")
    fa.fa_fwd(q, None, None, o, lse, 1, 2, 2, 5, 0, 64, False, 0.125, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(lse == float("-inf"))


def test_empty_batch_is_noop():
    from exact_tiled_attention_02_amd import fa
    fa.fa_fwd(None, None, None, None, None, 0, 4, 2, 16, 16, 64, True, 0.125)


def test_inputs_untouched_and_deterministic():
    """No entry point modifies its input ([FUSED07] task 07.2 checklist), and
    two runs give identical bits."""
    from exact_tiled_attention_02_amd import fa
    w = inputs.Prefill("t", B=1, Hq=4, Hkv=2, Tq=513, Tk=513, d=128, causal=True, seed=9)
    q, k, v = inputs.prefill_inputs(w)
    tq, tk, tv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    outs = []
    say("fa_fwd bf16 determinism")
    for _ in range(2):
        o = torch.empty(1, 4, 513, 128, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(1, 4, 513, device="cuda")
        fa.fa_fwd(tq, tk, tv, o, lse, 1, 4, 2, 513, 513, 128, True, w.scale)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(tq.view(torch.int16).cpu().numpy().view(np.uint16), q)
    assert np.array_equal(tk.view(torch.int16).cpu().numpy().view(np.uint16), k)
    assert np.array_equal(tv.view(torch.int16).cpu().numpy().view(np.uint16), v)


def test_gqa_equals_repeated_heads_on_gpu():
    """Any size property: GQA output equals MHA output on repeated kv heads."""
    w = inputs.Prefill("t", B=2, Hq=8, Hkv=2, Tq=333, Tk=333, d=64, causal=True, seed=10)
    q, k, v = inputs.prefill_inputs(w)
    say("fa_fwd bf16 gqa vs mha")
    O1, L1 = run_bf16(q, k, v, True, w.scale)
    O2, L2 = run_bf16(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), True, w.scale)
    check("O", O1, O2, BF16_O_TOL)
    check("lse", L1, L2, BF16_LSE_TOL)
