"""The decode test bound (gpu_helpers.decode_error_bound) against a CPU
emulation of the decode kernel's arithmetic: scores from exact bf16 products
summed in fp32, P = 2^(s c - m c) in fp32, l from the unrounded P, P rounded
to bf16 for an fp32 P.V sum, O rounded to bf16.  The faithful emulation stays
within the bound on every element; the same emulation with P rounded to 4
significant bits instead of 8 (a planted mistake about 10 times larger than
the kernel's rounding) leaves it."""
import numpy as np
import pytest

import oracle
from exact_tiled_attention_02_amd import inputs
from gpu_helpers import decode_error_bound


def round_sig(x, bits):
    """x rounded to `bits` significant bits (round half to even)."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e)


def emulate_decode(q, K, V, seqlens, p_bits=8):
    B, Hq, d = q.shape
    g = Hq // K.shape[1]
    c = np.float32(1.0 / np.sqrt(d) * np.log2(np.e))
    O = np.zeros((B, Hq, d))
    for b in range(B):
        n = int(seqlens[b])
        if n == 0:
            continue
        for h in range(Hq):
            k = K[b, h // g, :n].astype(np.float32)
            v = V[b, h // g, :n].astype(np.float32)
            s = k @ q[b, h].astype(np.float32)            # exact products, fp32 sums
            m = s.max()
            P = np.exp2((s * c - m * c).astype(np.float32)).astype(np.float32)
            l = P.sum(dtype=np.float32)
            Pr = round_sig(P, p_bits).astype(np.float32)
            acc = (Pr @ v).astype(np.float32)
            O[b, h] = round_sig(acc / l, 8)
    return O


@pytest.fixture(scope="module")
def case():
    w = inputs.Decode("t", B=3, Hq=8, Hkv=2, Tk_max=1500, d=128, seq_lo=1, seq_hi=1500, seed=71)
    q, kc, vc, sl = inputs.decode_inputs(w)
    sl = np.array([1500, 37, 1], np.int32)
    qf, K, V = oracle.as_f64(q), oracle.as_f64(kc), oracle.as_f64(vc)
    Or, _ = oracle.decode_attention(q, kc, vc, sl)
    return qf, K, V, sl, Or, decode_error_bound(qf, K, V, sl)


def test_faithful_emulation_within_decode_bound(case):
    qf, K, V, sl, Or, bound = case
    ratio = np.max(np.abs(emulate_decode(qf, K, V, sl) - Or) / bound)
    assert ratio <= 1.0, ratio


def test_coarser_probability_rounding_leaves_decode_bound(case):
    qf, K, V, sl, Or, bound = case
    ratio = np.max(np.abs(emulate_decode(qf, K, V, sl, p_bits=4) - Or) / bound)
    assert ratio > 1.0, ratio
