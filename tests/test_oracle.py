"""Pins for the CPU oracle: it is checked against values the pages print,
closed forms, invariants, a brute-force evaluation and an independent library
routine -- never against itself or the HIP path.

Page tags are those of the oracle package docstring.
"""
import math

import numpy as np
import pytest

import oracle
from exact_tiled_attention_02_amd import inputs

F64 = np.float64


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# Values the pages print
# ---------------------------------------------------------------------------

def test_fused07_worked_example(golden):
    """[FUSED07] 'Числовой пример: 8 токенов, блоки 4×4'."""
    g = golden("fused07_worked_example.json")
    s = np.array(g["scores_row0"], F64)
    v = np.array(g["values"], F64)
    tol = g["tolerance"]
    p = g["printed"]
    # Scores enter as scale * q * k with d = 1, q = 1, scale = 1.
    q = np.ones((1, 1, 1, 1))
    k = s.reshape(1, 1, 8, 1)
    vv = v.reshape(1, 1, 8, 1)

    # After block 1 only: m = 4, so l1 = exp(lse - 4) and O1 (unnormalised) = O * l1.
    O1, L1 = oracle.online_fold_attention(q, k[:, :, :4], vv[:, :, :4], causal=False,
                                          scale=1.0, Br=1, Bc=4)
    l1 = math.exp(L1[0, 0, 0] - p["block1"]["m"])
    assert abs(l1 - p["block1"]["l"]) < tol
    assert abs(O1[0, 0, 0, 0] * l1 - p["block1"]["O"]) < tol

    # After block 2: m = 5 and corr = exp(4 - 5).
    O2, L2 = oracle.online_fold_attention(q, k, vv, causal=False, scale=1.0, Br=1, Bc=4)
    l2 = math.exp(L2[0, 0, 0] - p["block2"]["m"])
    assert abs(l2 - p["block2"]["l"]) < tol
    assert abs(O2[0, 0, 0, 0] * l2 - p["block2"]["O"]) < tol
    assert abs(l1 * p["block2"]["corr"] - p["block2"]["l_old_rescaled"]) < tol
    assert abs(O2[0, 0, 0, 0] - p["O_over_l"]) < tol

    # The definition and the element-by-element recurrence give the same O/l.
    O3, _ = oracle.softmax_attention(q, k, vv, causal=False, scale=1.0)
    assert abs(O3[0, 0, 0, 0] - p["O_over_l"]) < tol
    m, l, a, o = oracle.online_weighted_sum(s, v)
    assert m == 5 and abs(l - p["block2"]["l"]) < tol and abs(o - p["O_over_l"]) < tol


def test_lesson_online_normalizer(golden):
    """[LESSON] 'Online softmax: нормировка за один проход', example x = (1, 3, 2)."""
    g = golden("lesson_online_normalizer.json")
    x, v = g["x"], g["v"]
    for n, step in enumerate(g["printed_steps"], start=1):
        m, l = oracle.online_normalizer(x[:n])
        assert m == step["m"]
        assert abs(l - step["l"]) <= 0.5e-4
        if step["factor"] is not None:
            m_prev, _ = oracle.online_normalizer(x[:n - 1])
            assert abs(math.exp(m_prev - m) - step["factor"]) <= 0.5e-4
    m, l, a, o = oracle.online_weighted_sum(x, v)
    fin = g["printed_final"]
    assert abs(a - fin["a"]) <= 0.5e-2
    assert abs(l - fin["l"]) <= 0.5e-4
    assert abs(o - fin["o"]) <= 0.5e-3
    # Probabilities e^{x - lse}, through the attention definition (d = 1).
    q = np.ones((1, 1, 1, 1))
    k = np.array(x, F64).reshape(1, 1, 3, 1)
    vv = np.array(v, F64).reshape(1, 1, 3, 1)
    O, L = oracle.softmax_attention(q, k, vv, causal=False, scale=1.0)
    probs = np.exp(np.array(x, F64) - L[0, 0, 0])
    assert np.all(np.abs(probs - g["printed_probabilities"]) <= 0.5e-3)
    assert abs(O[0, 0, 0, 0] - fin["o"]) <= 0.5e-3


def test_lesson_quiz_two_scores():
    """[LESSON] quiz 1: the row (2, 5) read online gives l = 1 + e^-3 at m = 5."""
    m, l = oracle.online_normalizer([2.0, 5.0])
    assert m == 5.0 and abs(l - (1 + math.exp(-3))) < 1e-15 and round(l, 2) == 1.05


def test_book5_example_5_6(golden):
    """[BOOK5] 5.3.3, Example 5-6: scores [0, ln 2], values [1, 3] -> 7/3."""
    g = golden("book5_example_5_6.json")
    s = np.array([0.0, math.log(2.0)])
    v = np.array(g["values"])
    m, l, a, o = oracle.online_weighted_sum(s, v)
    assert abs(l - g["printed"]["after_block2"]["l"]) < 1e-15
    assert abs(a - g["printed"]["after_block2"]["u"]) < 1e-15
    assert abs(o - 7 / 3) < 1e-15
    m1, l1, a1, _ = oracle.online_weighted_sum(s[:1], v[:1])
    assert (m1, l1, a1) == (0.0, 1.0, 1.0)
    q = np.ones((1, 1, 1, 1))
    k = s.reshape(1, 1, 2, 1)
    vv = v.reshape(1, 1, 2, 1)
    for O, _ in (oracle.softmax_attention(q, k, vv, causal=False, scale=1.0),
                 oracle.online_fold_attention(q, k, vv, causal=False, scale=1.0, Br=1, Bc=1)):
        assert abs(O[0, 0, 0, 0] - 7 / 3) < 1e-15
    # The same two blocks as a 2-way split-KV merge (decode form, d = 1 so
    # scale = 1 exactly).
    O, _ = oracle.decode_split_merge(q[:, :, 0], k, vv, np.array([2]), num_splits=2, tile=1)
    assert abs(O[0, 0, 0] - 7 / 3) < 1e-15


def test_causal_block_counts(golden):
    g = golden("causal_block_counts.json")
    for c in g["cases"]:
        assert oracle.causal_block_pairs(c["T"], c["T"], c["Br"], c["Bc"], False) == c["noncausal"]
        assert oracle.causal_block_pairs(c["T"], c["T"], c["Br"], c["Bc"], True) == c["causal"]
    for T, B in [(2048, 128), (4096, 64), (32768, 128), (256, 32)]:
        nb = T // B
        assert oracle.causal_block_pairs(T, T, B, B, True) == nb * (nb + 1) // 2
    # The fold visits exactly the pairs the count says (ragged tiles too).
    rng = np.random.default_rng(1)
    q, k, v = (_rand(rng, 1, 1, 37, 4) for _ in range(3))
    for causal in (False, True):
        _, _, pairs = oracle.online_fold_attention(q, k, v, causal=causal, scale=0.5,
                                                   Br=7, Bc=13, count=True)
        assert pairs == oracle.causal_block_pairs(37, 37, 7, 13, causal)


# ---------------------------------------------------------------------------
# Closed forms and invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    rng = np.random.default_rng(2)
    T, d = 29, 8
    q = np.zeros((1, 2, T, d))
    k = _rand(rng, 1, 1, T, d)
    v = _rand(rng, 1, 1, T, d)
    O, L = oracle.softmax_attention(q, k, v, causal=causal, scale=0.3)
    if causal:
        want = np.cumsum(v[0, 0], axis=0) / np.arange(1, T + 1)[:, None]
        want_l = np.log(np.arange(1, T + 1))
    else:
        want = np.broadcast_to(v[0, 0].mean(axis=0), (T, d))
        want_l = np.full(T, math.log(T))
    for h in range(2):
        assert np.max(np.abs(O[0, h] - want)) < 1e-14
        assert np.max(np.abs(L[0, h] - want_l)) < 1e-14


def test_constant_value_rows_give_that_row():
    rng = np.random.default_rng(3)
    q = _rand(rng, 2, 2, 17, 8, scale=3)
    k = _rand(rng, 2, 1, 17, 8)
    c = _rand(rng, 8)
    v = np.broadcast_to(c, (2, 1, 17, 8)).copy()
    for causal in (False, True):
        O, _ = oracle.softmax_attention(q, k, v, causal=causal, scale=0.4)
        assert np.max(np.abs(O - c)) < 1e-14


def test_causal_first_row_is_first_value():
    rng = np.random.default_rng(4)
    q, k, v = (_rand(rng, 1, 1, 10, 6) for _ in range(3))
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=0.7)
    assert np.array_equal(O[0, 0, 0], v[0, 0, 0])
    assert abs(L[0, 0, 0] - 0.7 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-15


def test_two_key_closed_form():
    """softmax over two scores is a logistic weight; lse is logaddexp."""
    rng = np.random.default_rng(5)
    q = _rand(rng, 1, 1, 5, 4)
    k = _rand(rng, 1, 1, 2, 4)
    v = _rand(rng, 1, 1, 2, 3)
    O, L = oracle.softmax_attention(q, k, v, causal=False, scale=0.9)
    for i in range(5):
        s0 = 0.9 * q[0, 0, i] @ k[0, 0, 0]
        s1 = 0.9 * q[0, 0, i] @ k[0, 0, 1]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        want = w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1]
        assert np.max(np.abs(O[0, 0, i] - want)) < 1e-14
        assert abs(L[0, 0, i] - np.logaddexp(s0, s1)) < 1e-14


def test_key_shift_invariance():
    """K -> K + 1 w^T shifts every score of row i by scale * q_i . w:
    O is unchanged and lse moves by that amount ([FUSED07] 'Online softmax:
    вывод': the normalised result does not depend on the constant subtracted)."""
    rng = np.random.default_rng(6)
    q, k, v = (_rand(rng, 1, 2, 21, 5) for _ in range(3))
    w = _rand(rng, 5)
    for causal in (False, True):
        O, L = oracle.softmax_attention(q, k, v, causal=causal, scale=0.6)
        O2, L2 = oracle.softmax_attention(q, k + w, v, causal=causal, scale=0.6)
        assert np.max(np.abs(O - O2)) < 1e-13
        assert np.max(np.abs(L2 - L - 0.6 * q @ w)) < 1e-13


def test_noncausal_key_permutation_invariance():
    rng = np.random.default_rng(7)
    q, k, v = (_rand(rng, 1, 1, 15, 4) for _ in range(3))
    perm = rng.permutation(15)
    O, L = oracle.softmax_attention(q, k, v, causal=False, scale=1.1)
    O2, L2 = oracle.softmax_attention(q, k[:, :, perm], v[:, :, perm], causal=False, scale=1.1)
    assert np.max(np.abs(O - O2)) < 1e-14 and np.max(np.abs(L - L2)) < 1e-14


def test_causal_prefix_consistency():
    rng = np.random.default_rng(8)
    q, k, v = (_rand(rng, 1, 1, 40, 4) for _ in range(3))
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=0.5)
    O2, L2 = oracle.softmax_attention(q[:, :, :23], k[:, :, :23], v[:, :, :23], causal=True, scale=0.5)
    assert np.max(np.abs(O[:, :, :23] - O2)) < 1e-14
    assert np.max(np.abs(L[:, :, :23] - L2)) < 1e-14


def test_gqa_equals_repeated_kv_heads():
    """Query head h reads kv head h // g: same as repeating each kv head g times
    (and different from the h % Hkv assignment)."""
    rng = np.random.default_rng(9)
    q = _rand(rng, 2, 8, 11, 4)
    k = _rand(rng, 2, 2, 11, 4)
    v = _rand(rng, 2, 2, 11, 4)
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=0.5)
    Om, Lm = oracle.softmax_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1),
                                      causal=True, scale=0.5)
    assert np.max(np.abs(O - Om)) < 1e-14 and np.max(np.abs(L - Lm)) < 1e-14
    Ow, _ = oracle.softmax_attention(q, np.tile(k, (1, 4, 1, 1)), np.tile(v, (1, 4, 1, 1)),
                                     causal=True, scale=0.5)
    assert np.max(np.abs(O - Ow)) > 1e-3


def test_brute_force_tiny():
    """Direct evaluation with Python floats: exp(s)/sum exp(s) without any max
    subtraction (safe at these magnitudes), explicit loops, explicit mask."""
    rng = np.random.default_rng(10)
    for (Tq, Tk, d, causal) in [(1, 1, 1, False), (3, 5, 2, False), (5, 5, 3, True),
                                (4, 6, 2, True), (6, 3, 3, True)]:
        q, k, v = _rand(rng, 1, 1, Tq, d), _rand(rng, 1, 1, Tk, d), _rand(rng, 1, 1, Tk, d)
        sc = 0.8
        O, L = oracle.softmax_attention(q, k, v, causal=causal, scale=sc)
        for i in range(Tq):
            num = [0.0] * d
            den = 0.0
            for j in range(Tk):
                if causal and j > i:
                    continue
                s = sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) * sc
                e = math.exp(s)
                den += e
                for t in range(d):
                    num[t] += e * v[0, 0, j, t]
            for t in range(d):
                assert abs(O[0, 0, i, t] - num[t] / den) < 1e-13
            assert abs(L[0, 0, i] - math.log(den)) < 1e-13


# ---------------------------------------------------------------------------
# Independent library routine: torch CPU SDPA (math backend) in fp64
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(1, 4, 2, 33, 33, 16, True), (2, 6, 3, 19, 40, 8, False),
                                   (1, 2, 2, 50, 50, 32, True), (1, 4, 1, 17, 9, 8, True)])
def test_matches_torch_sdpa_fp64(shape):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    rng = np.random.default_rng(11)
    q = _rand(rng, B, Hq, Tq, d, scale=2)
    k = _rand(rng, B, Hkv, Tk, d)
    v = _rand(rng, B, Hkv, Tk, d)
    sc = 1 / math.sqrt(d)
    O, L = oracle.softmax_attention(q, k, v, causal=causal, scale=sc)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=sc, enable_gqa=True)
    assert np.max(np.abs(O - ref.numpy())) < 1e-12
    # lse via torch.logsumexp of the masked score matrix (top-left causal tril).
    g = Hq // Hkv
    s = torch.matmul(tq, tk.repeat_interleave(g, dim=1).transpose(-1, -2)) * sc
    if causal:
        s = s.masked_fill(~torch.ones(Tq, Tk, dtype=torch.bool).tril(), float("-inf"))
    assert np.max(np.abs(L - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


# ---------------------------------------------------------------------------
# The two algorithmic routes agree (fp64 expects ~1e-16 per [LESSON]
# 'Почему ответ точный'; bound set at 1e-12)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Br,Bc", [(64, 64), (7, 13), (1, 1), (32, 16), (128, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_fold_matches_three_pass(Br, Bc, causal):
    rng = np.random.default_rng(12)
    q = _rand(rng, 2, 4, 100, 16, scale=3)
    k = _rand(rng, 2, 2, 100, 16)
    v = _rand(rng, 2, 2, 100, 16)
    O, L = oracle.softmax_attention(q, k, v, causal=causal, scale=0.25)
    O2, L2 = oracle.online_fold_attention(q, k, v, causal=causal, scale=0.25, Br=Br, Bc=Bc)
    assert np.max(np.abs(O - O2)) <= 1e-12
    assert np.max(np.abs(L - L2)) <= 1e-12


def test_fold_on_bf16_inputs_matches_three_pass():
    w = inputs.Prefill("t", B=1, Hq=4, Hkv=2, Tq=200, Tk=200, d=64, causal=True, q_mult=3.0)
    q, k, v = inputs.prefill_inputs(w)
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=w.scale)
    O2, L2 = oracle.online_fold_attention(q, k, v, causal=True, scale=w.scale, Br=64, Bc=64)
    assert np.max(np.abs(O - O2)) <= 1e-12 and np.max(np.abs(L - L2)) <= 1e-12


def test_large_query_scale_is_stable():
    """[FUSED07] task 07.2, requirement 4: Q x 100 must give finite numbers that
    agree with the reference."""
    rng = np.random.default_rng(13)
    q = _rand(rng, 1, 1, 64, 16, scale=100)
    k, v = _rand(rng, 1, 1, 64, 16), _rand(rng, 1, 1, 64, 16)
    for causal in (False, True):
        O, L = oracle.softmax_attention(q, k, v, causal=causal, scale=0.25)
        O2, L2 = oracle.online_fold_attention(q, k, v, causal=causal, scale=0.25, Br=16, Bc=16)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
        assert np.max(np.abs(O - O2)) <= 1e-12
        assert np.max(np.abs(L - L2)) / np.max(np.abs(L)) <= 1e-14


def test_rows_helper_matches_full():
    rng = np.random.default_rng(14)
    q = _rand(rng, 2, 4, 70, 8)
    k, v = _rand(rng, 2, 2, 70, 8), _rand(rng, 2, 2, 70, 8)
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=0.3, row_chunk=16)
    rows = [0, 5, 31, 69]
    Or, Lr = oracle.softmax_attention_rows(q, k, v, causal=True, scale=0.3, b=1, h=3, rows=rows)
    assert np.max(np.abs(Or - O[1, 3, rows])) < 1e-14
    assert np.max(np.abs(Lr - L[1, 3, rows])) < 1e-14


def test_empty_key_set():
    q = np.ones((1, 1, 3, 4))
    k = np.zeros((1, 1, 0, 4))
    v = np.zeros((1, 1, 0, 4))
    O, L = oracle.softmax_attention(q, k, v, causal=False, scale=1.0)
    assert np.all(O == 0) and np.all(L == -np.inf)


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def _small_decode(seed=15, B=5, Hq=8, Hkv=2, Tmax=300, d=16, poison=True):
    w = inputs.Decode("t", B=B, Hq=Hq, Hkv=Hkv, Tk_max=Tmax, d=d, seq_lo=1, seq_hi=Tmax, seed=seed)
    return inputs.decode_inputs(w, poison_tail=poison)


def test_decode_equals_single_row_prefill():
    q, kc, vc, sl = _small_decode(poison=False)
    O, L = oracle.decode_attention(q, kc, vc, sl)
    d = q.shape[-1]
    for b in range(q.shape[0]):
        n = sl[b]
        Op, Lp = oracle.softmax_attention(q[b:b + 1, :, None, :], kc[b:b + 1, :, :n],
                                          vc[b:b + 1, :, :n], causal=False, scale=1 / math.sqrt(d))
        assert np.max(np.abs(O[b] - Op[0, :, 0])) < 1e-14
        assert np.max(np.abs(L[b] - Lp[0, :, 0])) < 1e-14


def test_decode_ignores_cache_beyond_seqlen():
    q, kc, vc, sl = _small_decode(poison=True)
    O, L = oracle.decode_attention(q, kc, vc, sl)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


@pytest.mark.parametrize("S", [1, 2, 3, 7, 16, 64])
@pytest.mark.parametrize("tile", [1, 16, 64])
def test_decode_split_merge_matches_three_pass(S, tile):
    q, kc, vc, sl = _small_decode()
    O, L = oracle.decode_attention(q, kc, vc, sl)
    O2, L2 = oracle.decode_split_merge(q, kc, vc, sl, num_splits=S, tile=tile)
    assert np.max(np.abs(O - O2)) <= 1e-12 and np.max(np.abs(L - L2)) <= 1e-12


def test_decode_zero_length_sequence():
    q, kc, vc, sl = _small_decode()
    sl = sl.copy()
    sl[2] = 0
    for O, L in (oracle.decode_attention(q, kc, vc, sl),
                 oracle.decode_split_merge(q, kc, vc, sl, num_splits=4)):
        assert np.all(O[2] == 0) and np.all(L[2] == -np.inf)
        assert np.all(np.isfinite(O))


# ---------------------------------------------------------------------------
# Input generator
# ---------------------------------------------------------------------------

def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-9, 1 + 2**-7 + 2**-8, -2.5, 3.0e38, 1e-40,
                  np.float32(np.inf), -0.0], np.float32)
    bits = inputs.f32_to_bf16_bits(x)
    assert [hex(b) for b in bits] == ['0x3f80', '0x3f80', '0x3f81', '0x3f82', '0xc020',
                                      '0x7f62', '0x1', '0x7f80', '0x8000']
    nan = inputs.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0
    # Round-trip of representable values is exact; rounding error <= half ulp.
    rng = np.random.default_rng(0)
    y = rng.standard_normal(100000).astype(np.float32)
    r = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(y))
    ulp = np.spacing(np.abs(r).astype(np.float32)) * 65536
    assert np.all(np.abs(r - y) <= ulp / 2)
    assert np.array_equal(inputs.f32_to_bf16_bits(r), inputs.f32_to_bf16_bits(y))


def test_decode_seqlens_seed0():
    sl = inputs.decode_seqlens(inputs.FLASH_DECODE)
    assert sl.tolist() == [28027, 21244, 17250, 9588, 10796, 2324, 3412, 1548, 6587, 26841,
                           21639, 29999, 17011, 20281, 31840, 24181]
    assert int(sl.sum()) == 272568


# ---------------------------------------------------------------------------
# Backward pass ([LESSON] "Обратный проход: пересчитать дешевле, чем хранить")
# ---------------------------------------------------------------------------

BWD_SHAPES = [
    # B, Hq, Hkv, Tq, Tk, d, causal
    (1, 2, 2, 13, 13, 16, True),
    (2, 4, 2, 20, 17, 8, False),
    (1, 6, 2, 9, 30, 8, True),     # Tq < Tk, causal top-left
    (1, 2, 1, 30, 9, 8, True),     # Tq > Tk
    (1, 4, 1, 11, 11, 4, False),   # g = 4
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_matches_torch_autograd_fp64(shape):
    """Library routine: torch autograd in fp64 through the naive masked
    attention (the same check the lesson page runs)."""
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Tq, Tk, d, causal = shape
    rng = np.random.default_rng(11)
    q, k, v, do = (_rand(rng, B, Hq, Tq, d), _rand(rng, B, Hkv, Tk, d),
                   _rand(rng, B, Hkv, Tk, d), _rand(rng, B, Hq, Tq, d))
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    g = Hq // Hkv
    kk = tk.repeat_interleave(g, dim=1)
    vv = tv.repeat_interleave(g, dim=1)
    S = scale * (tq @ kk.transpose(-1, -2))
    if causal:
        mask = torch.ones(Tq, Tk, dtype=torch.bool).tril()
        S = S.masked_fill(~mask, float("-inf"))
    O = torch.softmax(S, dim=-1) @ vv
    O.backward(torch.tensor(do))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=causal, scale=scale)
    assert np.max(np.abs(dq - tq.grad.numpy())) < 1e-12
    assert np.max(np.abs(dk - tk.grad.numpy())) < 1e-12
    assert np.max(np.abs(dv - tv.grad.numpy())) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    """Brute force: central differences of f(x) = <dO, O(x)> through the
    forward oracle along random directions equal <grad, direction>."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, T, d = 1, 2, 1, 6, 4
    q, k, v, do = (_rand(rng, B, Hq, T, d), _rand(rng, B, Hkv, T, d),
                   _rand(rng, B, Hkv, T, d), _rand(rng, B, Hq, T, d))
    scale = 0.7
    grads = oracle.attention_backward(q, k, v, do, causal=causal, scale=scale)

    def f(qq, kk, vv):
        O, _ = oracle.softmax_attention(qq, kk, vv, causal=causal, scale=scale)
        return float(np.sum(do * O))

    eps = 1e-6
    for which in range(3):
        for _ in range(3):
            args = [q.copy(), k.copy(), v.copy()]
            direction = _rand(rng, *args[which].shape)
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which] += eps * direction
            minus[which] -= eps * direction
            fd = (f(*plus) - f(*minus)) / (2 * eps)
            assert abs(fd - float(np.sum(grads[which] * direction))) < 1e-7


def test_backward_invariants():
    """Shifting every key by one vector leaves O unchanged, so the key
    gradients of a head sum to zero; the row term rowsum(P * dP) equals
    dO . O (the identity the lesson uses); dO = 0 gives zero gradients."""
    rng = np.random.default_rng(13)
    B, Hq, Hkv, T, d = 2, 4, 2, 24, 8
    q, k, v, do = (_rand(rng, B, Hq, T, d), _rand(rng, B, Hkv, T, d),
                   _rand(rng, B, Hkv, T, d), _rand(rng, B, Hq, T, d))
    for causal in (False, True):
        dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=causal, scale=0.35)
        assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
        z = oracle.attention_backward(q, k, v, np.zeros_like(do), causal=causal, scale=0.35)
        assert all(np.all(x == 0) for x in z)
    # D identity on one head, P recovered by using V = identity.
    Tk = T
    eye = np.eye(Tk).reshape(1, 1, Tk, Tk)
    qq, kk = q[:1, :1], k[:1, :1]
    P, _ = oracle.softmax_attention(qq, kk, eye, causal=True, scale=0.35)
    O, _ = oracle.softmax_attention(qq, kk, v[:1, :1], causal=True, scale=0.35)
    dP = do[0, 0] @ v[0, 0].T
    assert np.max(np.abs((P[0, 0] * dP).sum(axis=1) - (do[0, 0] * O[0, 0]).sum(axis=1))) < 1e-12


def test_backward_dv_closed_form():
    """dO = all ones: dV_j = (sum_i P_ij) * ones -- the column sums of the
    probabilities, obtained independently through the forward oracle with
    V = identity."""
    rng = np.random.default_rng(14)
    T, d = 16, 8
    q, k, v = _rand(rng, 1, 1, T, d), _rand(rng, 1, 1, T, d), _rand(rng, 1, 1, T, d)
    P, _ = oracle.softmax_attention(q, k, np.eye(T).reshape(1, 1, T, T), causal=True, scale=0.4)
    _, _, dv = oracle.attention_backward(q, k, v, np.ones((1, 1, T, d)), causal=True, scale=0.4)
    colsum = P[0, 0].sum(axis=0)
    assert np.max(np.abs(dv[0, 0] - colsum[:, None])) < 1e-12


# ---------------------------------------------------------------------------
# Bottom-right causal alignment (chunked prefill over a cache)
# ---------------------------------------------------------------------------

BR_SHAPES = [
    # B, Hq, Hkv, Tq, Tk, d
    (1, 4, 2, 7, 30, 8),
    (2, 2, 2, 16, 16, 8),
    (1, 6, 3, 1, 25, 16),
    (1, 4, 1, 33, 70, 4),
]


@pytest.mark.parametrize("shape", BR_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bottom_right_matches_torch_lower_right(shape):
    """Library routine: torch fp64 SDPA with its lower-right causal bias."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right
    B, Hq, Hkv, Tq, Tk, d = shape
    rng = np.random.default_rng(31)
    q, k, v = _rand(rng, B, Hq, Tq, d, scale=2), _rand(rng, B, Hkv, Tk, d), _rand(rng, B, Hkv, Tk, d)
    sc = 1 / math.sqrt(d)
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=sc, align="bottom_right")
    g = Hq // Hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(Tq, Tk), scale=sc)
    assert np.max(np.abs(O - ref.numpy())) < 1e-12
    mask = causal_lower_right(Tq, Tk)._materialize()
    s = (tq @ tk.transpose(-1, -2) * sc).masked_fill(~mask, float("-inf"))
    assert np.max(np.abs(L - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


def test_bottom_right_equals_top_left_when_square():
    rng = np.random.default_rng(32)
    q, k, v = _rand(rng, 1, 2, 20, 8), _rand(rng, 1, 2, 20, 8), _rand(rng, 1, 2, 20, 8)
    a = oracle.softmax_attention(q, k, v, causal=True, scale=0.3)
    b = oracle.softmax_attention(q, k, v, causal=True, scale=0.3, align="bottom_right")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bottom_right_is_the_tail_of_full_causal():
    """A chunk of the last Tq query rows against the whole sequence's keys
    gives the last Tq rows of the full causal (top-left) result."""
    rng = np.random.default_rng(33)
    T, Tq = 45, 12
    q, k, v = _rand(rng, 1, 4, T, 8, scale=2), _rand(rng, 1, 2, T, 8), _rand(rng, 1, 2, T, 8)
    Of, Lf = oracle.softmax_attention(q, k, v, causal=True, scale=0.35)
    Oc, Lc = oracle.softmax_attention(q[:, :, T - Tq:], k, v, causal=True, scale=0.35,
                                      align="bottom_right")
    assert np.max(np.abs(Oc - Of[:, :, T - Tq:])) < 1e-14
    assert np.max(np.abs(Lc - Lf[:, :, T - Tq:])) < 1e-14
    dq_f, _, _ = oracle.attention_backward(q, k, v, q * 0 + 1, causal=True, scale=0.35)
    dq_c, _, _ = oracle.attention_backward(q[:, :, T - Tq:], k, v, (q * 0 + 1)[:, :, T - Tq:],
                                           causal=True, scale=0.35, align="bottom_right")
    assert np.max(np.abs(dq_c - dq_f[:, :, T - Tq:])) < 1e-13


def test_bottom_right_more_rows_than_keys():
    """Tq > Tk: the first Tq - Tk rows see no key (O = 0, lse = -inf); row
    Tq - Tk + i sees keys 0..i, i.e. the top-left result of the later rows."""
    rng = np.random.default_rng(34)
    q, k, v = _rand(rng, 1, 2, 30, 8), _rand(rng, 1, 1, 12, 8), _rand(rng, 1, 1, 12, 8)
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=0.4, align="bottom_right")
    assert np.all(O[:, :, :18] == 0) and np.all(L[:, :, :18] == -np.inf)
    Ot, Lt = oracle.softmax_attention(q[:, :, 18:], k, v, causal=True, scale=0.4)
    assert np.max(np.abs(O[:, :, 18:] - Ot)) < 1e-14 and np.max(np.abs(L[:, :, 18:] - Lt)) < 1e-14
    Of, Lf = oracle.online_fold_attention(q, k, v, causal=True, scale=0.4, Br=7, Bc=5,
                                          align="bottom_right")
    assert np.max(np.abs(Of - O)) < 1e-12
    assert np.all(Lf[:, :, :18] == -np.inf) and np.max(np.abs(Lf[:, :, 18:] - L[:, :, 18:])) < 1e-12


@pytest.mark.parametrize("Br,Bc", [(64, 64), (7, 13), (1, 1)])
def test_bottom_right_fold_and_rows_match_three_pass(Br, Bc):
    rng = np.random.default_rng(35)
    q, k, v = _rand(rng, 1, 4, 37, 16, scale=3), _rand(rng, 1, 2, 90, 16), _rand(rng, 1, 2, 90, 16)
    O, L = oracle.softmax_attention(q, k, v, causal=True, scale=0.25, align="bottom_right")
    Of, Lf, pairs = oracle.online_fold_attention(q, k, v, causal=True, scale=0.25, Br=Br, Bc=Bc,
                                                 count=True, align="bottom_right")
    assert np.max(np.abs(O - Of)) < 1e-12 and np.max(np.abs(L - Lf)) < 1e-12
    rows = [0, 5, 36]
    Or, Lr = oracle.softmax_attention_rows(q, k, v, causal=True, scale=0.25, b=0, h=3, rows=rows,
                                           align="bottom_right")
    assert np.max(np.abs(Or - O[0, 3, rows])) < 1e-14 and np.max(np.abs(Lr - L[0, 3, rows])) < 1e-14


def test_decode_is_bottom_right_single_row():
    """One new token over a cache of n keys is bottom-right attention with
    Tq = 1 (it sees every cached key)."""
    q, kc, vc, sl = _small_decode(poison=False)
    O, L = oracle.decode_attention(q, kc, vc, sl)
    d = q.shape[-1]
    for b in range(q.shape[0]):
        n = sl[b]
        Op, Lp = oracle.softmax_attention(q[b:b + 1, :, None, :], kc[b:b + 1, :, :n],
                                          vc[b:b + 1, :, :n], causal=True, scale=1 / math.sqrt(d),
                                          align="bottom_right")
        assert np.max(np.abs(O[b] - Op[0, :, 0])) < 1e-14
        assert np.max(np.abs(L[b] - Lp[0, :, 0])) < 1e-14


@pytest.mark.parametrize("shape", [(1, 4, 2, 7, 19, 8), (1, 2, 1, 13, 13, 4)],
                         ids=lambda s: "x".join(map(str, s)))
def test_backward_bottom_right_matches_torch_autograd(shape):
    torch = pytest.importorskip("torch")
    from torch.nn.attention.bias import causal_lower_right
    B, Hq, Hkv, Tq, Tk, d = shape
    rng = np.random.default_rng(36)
    q, k, v, do = (_rand(rng, B, Hq, Tq, d), _rand(rng, B, Hkv, Tk, d),
                   _rand(rng, B, Hkv, Tk, d), _rand(rng, B, Hq, Tq, d))
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    g = Hq // Hkv
    S = scale * (tq @ tk.repeat_interleave(g, dim=1).transpose(-1, -2))
    S = S.masked_fill(~causal_lower_right(Tq, Tk)._materialize(), float("-inf"))
    O = torch.softmax(S, dim=-1) @ tv.repeat_interleave(g, dim=1)
    O.backward(torch.tensor(do))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=True, scale=scale,
                                           align="bottom_right")
    assert np.max(np.abs(dq - tq.grad.numpy())) < 1e-12
    assert np.max(np.abs(dk - tk.grad.numpy())) < 1e-12
    assert np.max(np.abs(dv - tv.grad.numpy())) < 1e-12


def test_causal_offset_values():
    assert oracle.causal_offset(5, 9, "top_left") == 0
    assert oracle.causal_offset(5, 9, "bottom_right") == 4
    assert oracle.causal_offset(9, 5, "bottom_right") == -4
    with pytest.raises(ValueError):
        oracle.causal_offset(1, 1, "middle")


# ---------------------------------------------------------------------------
# Decode over an 8-bit (E4M3, per-row scale) cache
# ---------------------------------------------------------------------------

def test_e4m3_decoder_matches_torch_all_codes():
    """Library routine: torch's float8_e4m3fn widening of all 256 codes."""
    torch = pytest.importorskip("torch")
    c = np.arange(256, dtype=np.uint8)
    a = oracle.e4m3_to_f64(c)
    b = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_e4m3_format_values():
    """Values fixed by the format: zero, one, the extremes, subnormals, NaN."""
    v = oracle.e4m3_to_f64(np.array([0x00, 0x80, 0x38, 0xB8, 0x7E, 0xFE, 0x01, 0x07, 0x08, 0x40,
                                     0x7F, 0xFF], np.uint8))
    assert v[0] == 0 and v[1] == 0 and math.copysign(1, v[1]) == -1
    assert v[2] == 1.0 and v[3] == -1.0
    assert v[4] == 448.0 and v[5] == -448.0
    assert v[6] == 2.0 ** -9 and v[7] == 7 * 2.0 ** -9 and v[8] == 2.0 ** -6
    assert v[9] == 2.0
    assert np.isnan(v[10]) and np.isnan(v[11])


def _small_fp8_decode(poison=False):
    w = inputs.Decode("t", B=3, Hq=8, Hkv=2, Tk_max=70, d=16, seq_lo=0, seq_hi=70, seed=5,
                      kv_dtype="fp8")
    return inputs.decode_inputs_fp8(w, poison_tail=poison)


def test_fp8_decode_is_decode_of_the_dequantized_cache():
    """Dequantised with torch's E4M3 widening times the row scales, the cache
    gives the same result through the plain decode definition."""
    torch = pytest.importorskip("torch")
    q, kc, vc, ks, vs, sl = _small_fp8_decode()
    O, L = oracle.decode_attention_fp8(q, kc, vc, ks, vs, sl)
    K = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * ks[..., None]
    V = torch.from_numpy(vc).view(torch.float8_e4m3fn).to(torch.float64).numpy() * vs[..., None]
    Or, Lr = oracle.decode_attention(q, K, V, sl)
    assert np.array_equal(np.isinf(L), np.isinf(Lr))
    assert np.max(np.abs(O - Or)) < 1e-14
    fin = np.isfinite(Lr)
    assert np.max(np.abs(L[fin] - Lr[fin])) < 1e-14


def test_fp8_decode_ignores_cache_beyond_seqlen():
    q, kc, vc, ks, vs, sl = _small_fp8_decode(poison=False)
    O, L = oracle.decode_attention_fp8(q, kc, vc, ks, vs, sl)
    q2, kc2, vc2, ks2, vs2, sl2 = _small_fp8_decode(poison=True)
    O2, L2 = oracle.decode_attention_fp8(q2, kc2, vc2, ks2, vs2, sl2)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_fp8_row_quantisation_uses_the_full_range():
    """Input side: every stored row's largest code is +-448 (amax scaling),
    and scale * code reproduces the drawn value to E4M3 precision."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 7, 32)).astype(np.float32)
    codes, sc = inputs.quantize_rows_e4m3(x)
    vals = oracle.e4m3_to_f64(codes)
    assert np.all(np.max(np.abs(vals), axis=-1) == 448.0)
    rel = np.abs(vals * sc[..., None] - x) / np.max(np.abs(x), axis=-1, keepdims=True)
    assert np.max(rel) <= 16 / 448   # half the E4M3 spacing (32) of the top binade, relative to amax


# ---------------------------------------------------------------------------
# Decode over an int8 (two's-complement codes, per-row scale) cache
# ---------------------------------------------------------------------------

def test_int8_decoder_matches_torch_all_codes():
    """Library routine: torch's reinterpretation of the 256 bytes as int8."""
    torch = pytest.importorskip("torch")
    c = np.arange(256, dtype=np.uint8)
    a = oracle.int8_to_f64(c)
    b = torch.from_numpy(c).view(torch.int8).to(torch.float64).numpy()
    assert np.array_equal(a, b)


def test_int8_format_values():
    """Values fixed by two's complement: 0, +1, the extremes, -1."""
    v = oracle.int8_to_f64(np.array([0x00, 0x01, 0x7F, 0x80, 0x81, 0xFF], np.uint8))
    assert list(v) == [0.0, 1.0, 127.0, -128.0, -127.0, -1.0]


def _small_int8_decode(poison=False):
    w = inputs.Decode("t", B=3, Hq=8, Hkv=2, Tk_max=70, d=16, seq_lo=0, seq_hi=70, seed=6,
                      kv_dtype="int8")
    return inputs.decode_inputs_int8(w, poison_tail=poison)


def test_int8_decode_is_decode_of_the_dequantized_cache():
    """Dequantised with torch's int8 view times the row scales, the cache
    gives the same result through the plain decode definition."""
    torch = pytest.importorskip("torch")
    q, kc, vc, ks, vs, sl = _small_int8_decode()
    O, L = oracle.decode_attention_int8(q, kc, vc, ks, vs, sl)
    K = torch.from_numpy(kc).view(torch.int8).to(torch.float64).numpy() * ks[..., None]
    V = torch.from_numpy(vc).view(torch.int8).to(torch.float64).numpy() * vs[..., None]
    Or, Lr = oracle.decode_attention(q, K, V, sl)
    assert np.array_equal(np.isinf(L), np.isinf(Lr))
    assert np.max(np.abs(O - Or)) < 1e-14
    fin = np.isfinite(Lr)
    assert np.max(np.abs(L[fin] - Lr[fin])) < 1e-14


def test_int8_decode_ignores_cache_beyond_seqlen():
    q, kc, vc, ks, vs, sl = _small_int8_decode(poison=False)
    O, L = oracle.decode_attention_int8(q, kc, vc, ks, vs, sl)
    q2, kc2, vc2, ks2, vs2, sl2 = _small_int8_decode(poison=True)
    assert np.any(kc2 != kc)
    O2, L2 = oracle.decode_attention_int8(q2, kc2, vc2, ks2, vs2, sl2)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_int8_row_quantisation_uses_the_full_range():
    """Input side: every stored row's largest code is +-127 (amax scaling),
    no code is -128, and scale * code is within half a step of the drawn
    value."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((5, 7, 32)).astype(np.float32)
    codes, sc = inputs.quantize_rows_int8(x)
    vals = oracle.int8_to_f64(codes)
    assert np.all(np.max(np.abs(vals), axis=-1) == 127.0)
    assert not np.any(codes == 0x80)
    err = np.abs(vals * sc[..., None] - x) / sc[..., None]
    assert np.max(err) <= 0.5 + 1e-5


def test_fp8_attention_inputs_dequantise_with_torch():
    """Library routine: torch's E4M3 widening times the block scales (per
    query row; per batch and kv head for k and v)."""
    torch = pytest.importorskip("torch")
    w = inputs.Prefill("t", B=2, Hq=4, Hkv=2, Tq=9, Tk=11, d=16, causal=True, q_mult=3.0, seed=40)
    q8, k8, v8, qs, ks, vs = inputs.prefill_inputs_fp8(w)
    q, k, v = oracle.fp8_attention_inputs(q8, k8, v8, qs, ks, vs)
    wid = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()  # noqa: E731
    assert np.array_equal(q, wid(q8) * qs[..., None])
    assert np.array_equal(k, wid(k8) * ks[:, :, None, None])
    assert np.array_equal(v, wid(v8) * vs[:, :, None, None])
    # Block scaling: each block's largest code is +-448.
    assert np.all(np.max(np.abs(wid(q8)), axis=-1) == 448)
    assert np.all(np.max(np.abs(wid(k8)), axis=(-1, -2)) == 448)
    # The stored values reproduce the fp32 draw within half an E4M3 step.
    rng = np.random.default_rng(40)
    qf = rng.standard_normal((2, 4, 9, 16), dtype=np.float32) * np.float32(3.0)
    assert np.max(np.abs(q - qf) / np.max(np.abs(qf), axis=-1, keepdims=True)) <= 16 / 448
