"""fa_decode_noalloc (decode with its workspace in the library's fixed device
array, for callers that cannot allocate) against fa_decode through the C
ABI: two calls in a row, the second smaller, each bitwise equal to fa_decode
with the same split count and within the bf16 bar of the oracle; a call whose
workspace would not fit is refused with FA_ERR_SCRATCH."""
import numpy as np
import pytest

import oracle
from exact_tiled_attention_02_amd import inputs
from gpu_helpers import check_bounded, decode_error_bound, dev_bf16, host_bf16_as_f64, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_02_amd import fa
    fa.load()


def _case(B, Hq, Hkv, Tmax, d, seed):
    w = inputs.Decode("t", B=B, Hq=Hq, Hkv=Hkv, Tk_max=Tmax, d=d, seq_lo=1, seq_hi=Tmax, seed=seed)
    q, kc, vc, sl = inputs.decode_inputs(w, poison_tail=True)
    sl[0] = 0   # one empty sequence
    kc[0] = inputs.BF16_NAN
    vc[0] = inputs.BF16_NAN
    return q, kc, vc, sl


def _both(q, kc, vc, sl, num_splits):
    """(fa_decode output, fa_decode_noalloc output) as bf16 bit patterns."""
    from exact_tiled_attention_02_amd import fa
    B, Hq, d = q.shape
    Hkv, Tmax = kc.shape[1], kc.shape[2]
    tq, tk, tv = dev_bf16(q), dev_bf16(kc), dev_bf16(vc)
    tsl = torch.from_numpy(np.ascontiguousarray(sl, np.int32)).cuda()
    stream = torch.cuda.current_stream()
    o_ref = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    o_na = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.fa_decode(tq, tk, tv, tsl, o_ref, B, Hq, Hkv, Tmax, d, num_splits, stream)
    fa.fa_decode_noalloc(tq, tk, tv, tsl, o_na, B, Hq, Hkv, Tmax, d, num_splits, stream)
    torch.cuda.synchronize()
    return o_ref, o_na


@pytest.mark.parametrize("num_splits", [0, 96])
def test_noalloc_matches_decode_on_two_calls(num_splits):
    cases = [(16, 32, 8, 3000, 128, 61), (3, 8, 2, 600, 64, 62)]   # the second is smaller
    for B, Hq, Hkv, Tmax, d, seed in cases:
        q, kc, vc, sl = _case(B, Hq, Hkv, Tmax, d, seed)
        say("fa_decode_noalloc vs fa_decode", (B, Hq, Hkv, Tmax, d), "splits", num_splits)
        o_ref, o_na = _both(q, kc, vc, sl, num_splits)
        a = o_ref.view(torch.int16).cpu().numpy()
        b = o_na.view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b), "fa_decode_noalloc differs from fa_decode"
        Or, _ = oracle.decode_attention(q, kc, vc, sl)
        check_bounded("O", host_bf16_as_f64(o_na), Or,
                      decode_error_bound(oracle.as_f64(q), oracle.as_f64(kc), oracle.as_f64(vc), sl))
        assert np.all(host_bf16_as_f64(o_na)[0] == 0)


def test_noalloc_refuses_oversized_workspace():
    """A split count whose partials exceed the fixed array is refused before
    anything is enqueued; the outputs stay untouched."""
    from exact_tiled_attention_02_amd import fa
    B, Hq, Hkv, Tmax, d = 2, 8, 2, 256, 128
    q, kc, vc, sl = _case(B, Hq, Hkv, Tmax, d, 63)
    tq, tk, tv = dev_bf16(q), dev_bf16(kc), dev_bf16(vc)
    tsl = torch.from_numpy(np.ascontiguousarray(sl, np.int32)).cuda()
    o = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    slot = 4 * (d + 2) * 4   # bytes per key range at four query heads per workgroup
    splits = fa.DECODE_SCRATCH_BYTES // slot + 1
    say("fa_decode_noalloc oversized, splits", splits)
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_noalloc(tq, tk, tv, tsl, o, B, Hq, Hkv, Tmax, d, splits,
                             torch.cuda.current_stream())
    assert e.value.status == fa.STATUS_CODES["FA_ERR_SCRATCH"]
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    # The same request through fa_decode (which grows its own workspace) works.
    fa.fa_decode(tq, tk, tv, tsl, o, B, Hq, Hkv, Tmax, d, splits, torch.cuda.current_stream())
    torch.cuda.synchronize()
    Or, _ = oracle.decode_attention(q, kc, vc, sl)
    check_bounded("O", host_bf16_as_f64(o), Or,
                  decode_error_bound(oracle.as_f64(q), oracle.as_f64(kc), oracle.as_f64(vc), sl))
