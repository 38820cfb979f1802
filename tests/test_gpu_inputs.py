"""No entry point modifies its input ([FUSED07] task 07.2 checklist) and each
is deterministic: fa_fwd_f32, fa_fwd_fp8, fa_decode, fa_decode_noalloc,
fa_decode_fp8 and fa_decode_int8 are each called twice through the C ABI;
every input buffer (tensors, scales, sequence lengths) must hold the same
bytes afterwards, and the two calls must give identical output bits.
(fa_fwd and fa_bwd have the same checks in their own test files.)"""
import numpy as np
import pytest

from exact_tiled_attention_02_amd import inputs
from gpu_helpers import dev_bf16, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_02_amd import fa
    fa.load()


def _dev(x):
    """Host array to a device tensor holding the same bytes (bf16 patterns
    arrive as uint16 and stay 2-byte integers)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return dev_bf16(x)
    return torch.from_numpy(x).cuda()


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().copy()


def _twice(name, ins, outs, call):
    """Run `call` twice; inputs unchanged, outputs bitwise equal."""
    before = [_bytes(t) for t in ins]
    runs = []
    for _ in range(2):
        for o in outs:
            o.fill_(float("nan")) if o.is_floating_point() else o.zero_()
        call(torch.cuda.current_stream())
        torch.cuda.synchronize()
        runs.append([_bytes(o) for o in outs])
    for i, (a, b) in enumerate(zip(before, [_bytes(t) for t in ins])):
        assert np.array_equal(a, b), f"{name}: input {i} was modified"
    for i, (a, b) in enumerate(zip(*runs)):
        assert np.array_equal(a, b), f"{name}: output {i} differs between two calls"


def test_forwards_leave_inputs_and_repeat_bitwise():
    from exact_tiled_attention_02_amd import fa
    w = inputs.Prefill("t", B=2, Hq=4, Hkv=2, Tq=190, Tk=257, d=64, causal=False, dtype="f32",
                       seed=301)
    q, k, v = (_dev(x) for x in inputs.prefill_inputs(w))
    o = torch.empty((w.B, w.Hq, w.Tq, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Tq), dtype=torch.float32, device="cuda")
    say("inputs: fa_fwd_f32")
    _twice("fa_fwd_f32", [q, k, v], [o, lse],
           lambda s: fa.fa_fwd_f32(q, k, v, o, lse, w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, False,
                                   w.scale, s))

    w8 = inputs.Prefill("t8", B=1, Hq=8, Hkv=2, Tq=300, Tk=300, d=128, causal=True, seed=302)
    ins8 = [_dev(x) for x in inputs.prefill_inputs_fp8(w8)]
    o8 = torch.empty((w8.B, w8.Hq, w8.Tq, w8.d), dtype=torch.bfloat16, device="cuda")
    lse8 = torch.empty((w8.B, w8.Hq, w8.Tq), dtype=torch.float32, device="cuda")
    say("inputs: fa_fwd_fp8")
    _twice("fa_fwd_fp8", ins8, [o8, lse8],
           lambda s: fa.fa_fwd_fp8(*ins8, o8, lse8, w8.B, w8.Hq, w8.Hkv, w8.Tq, w8.Tk, w8.d, True,
                                   w8.scale, s))


@pytest.mark.parametrize("kind", ["bf16", "noalloc", "fp8", "int8"])
def test_decodes_leave_inputs_and_repeat_bitwise(kind):
    from exact_tiled_attention_02_amd import fa
    w = inputs.Decode("t", B=6, Hq=16, Hkv=4, Tk_max=900, d=128, seq_lo=1, seq_hi=900, seed=310)
    o = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    say("inputs: decode", kind)
    if kind in ("bf16", "noalloc"):
        q, kc, vc, sl = inputs.decode_inputs(w, poison_tail=True)
        ins = [_dev(q), _dev(kc), _dev(vc), _dev(np.asarray(sl, np.int32))]
        fn = fa.fa_decode if kind == "bf16" else fa.fa_decode_noalloc
        _twice(kind, ins, [o], lambda s: fn(*ins, o, w.B, w.Hq, w.Hkv, w.Tk_max, w.d, 0, s))
    else:
        make = inputs.decode_inputs_fp8 if kind == "fp8" else inputs.decode_inputs_int8
        q, kc, vc, ks, vs, sl = make(w, poison_tail=True)
        ins = [_dev(q), _dev(kc), _dev(vc), _dev(np.asarray(ks, np.float32)),
               _dev(np.asarray(vs, np.float32)), _dev(np.asarray(sl, np.int32))]
        fn = fa.fa_decode_fp8 if kind == "fp8" else fa.fa_decode_int8
        _twice(kind, ins, [o], lambda s: fn(*ins, o, w.B, w.Hq, w.Hkv, w.Tk_max, w.d, 0, s))
