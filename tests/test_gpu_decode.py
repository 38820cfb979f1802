"""GPU parity of split-KV flash-decoding (fa_decode) against the fp64 CPU
oracle, through the C ABI.  Bar: every output element within
gpu_helpers.decode_error_bound, derived from the kernel's arithmetic (bf16
rounding of P and of O, fp32 scores and sums); two kernel results of the
same inputs differ by at most twice that bound."""
import math

import numpy as np
import pytest

import oracle
from exact_tiled_attention_02_amd import inputs
from gpu_helpers import (check_bounded, decode_error_bound, dev_bf16, host_bf16_as_f64, max_err,
                         say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_02_amd import fa
    fa.load()


def bound_of(q, kc, vc, sl):
    return decode_error_bound(oracle.as_f64(q), oracle.as_f64(kc), oracle.as_f64(vc), sl)


def run_decode(q, kc, vc, seqlens, num_splits):
    from exact_tiled_attention_02_amd import fa
    B, Hq, d = q.shape
    _, Hkv, Tmax, _ = kc.shape
    tq, tk, tv = dev_bf16(q), dev_bf16(kc), dev_bf16(vc)
    sl = torch.from_numpy(np.ascontiguousarray(seqlens, dtype=np.int32)).cuda()
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    fa.fa_decode(tq, tk, tv, sl, o, B, Hq, Hkv, Tmax, d, num_splits, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return host_bf16_as_f64(o)


SMALL = [
    # B, Hq, Hkv, Tmax, d, seqlens
    (3, 4, 1, 200, 128, [1, 64, 200]),
    (4, 8, 2, 300, 64, [0, 63, 65, 129]),
    (2, 32, 8, 1000, 128, [999, 1000]),
    (5, 6, 2, 257, 128, [257, 1, 128, 127, 200]),      # g = 3
    (2, 8, 1, 513, 64, [513, 300]),                    # g = 8
    (2, 2, 2, 96, 128, [96, 40]),                      # g = 1
    (2, 16, 1, 150, 128, [150, 77]),                   # g = 16: two head groups per kv head
    (2, 12, 1, 90, 64, [90, 1]),                       # g = 12: three groups of 4
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:5])))
@pytest.mark.parametrize("num_splits", [0, 1, 2, 7, 64])
def test_decode_small(case, num_splits):
    B, Hq, Hkv, Tmax, d, seqlens = case
    w = inputs.Decode("t", B=B, Hq=Hq, Hkv=Hkv, Tk_max=Tmax, d=d, seq_lo=1, seq_hi=Tmax, seed=21)
    q, kc, vc, _ = inputs.decode_inputs(w)
    sl = np.array(seqlens, np.int32)
    for b, n in enumerate(sl):   # every slot past the valid prefix is NaN
        kc[b, :, n:] = inputs.BF16_NAN
        vc[b, :, n:] = inputs.BF16_NAN
    say("fa_decode", case, "splits", num_splits)
    O = run_decode(q, kc, vc, sl, num_splits)
    Or, _ = oracle.decode_attention(q, kc, vc, sl)
    check_bounded("O", O, Or, bound_of(q, kc, vc, sl))
    for b, n in enumerate(sl):
        if n == 0:
            assert np.all(O[b] == 0)


@pytest.fixture(scope="module")
def flash_decode_case():
    w = inputs.FLASH_DECODE
    say("generating", w.name)
    q, kc, vc, sl = inputs.decode_inputs(w, poison_tail=True)
    Or, _ = oracle.decode_attention(q, kc, vc, sl)
    return q, kc, vc, sl, Or, bound_of(q, kc, vc, sl)


@pytest.mark.parametrize("num_splits", [0, 1, 8, 16, 32, 64])
def test_flash_decode_workload_full(flash_decode_case, num_splits):
    """B=16, Hq=32, Hkv=8, d=128, seqlens U[1024, 32768] (seed 0), cache
    poisoned with NaN past every valid prefix; every output element."""
    q, kc, vc, sl, Or, bound = flash_decode_case
    say("fa_decode", inputs.FLASH_DECODE.name, "splits", num_splits)
    O = run_decode(q, kc, vc, sl, num_splits)
    check_bounded("O", O, Or, bound)


def test_decode_deterministic_and_split_independent():
    w = inputs.Decode("t", B=4, Hq=8, Hkv=2, Tk_max=2000, d=128, seq_lo=1, seq_hi=2000, seed=22)
    q, kc, vc, sl = inputs.decode_inputs(w)
    say("fa_decode determinism")
    a = run_decode(q, kc, vc, sl, 5)
    b = run_decode(q, kc, vc, sl, 5)
    assert np.array_equal(a, b)
    c = run_decode(q, kc, vc, sl, 31)
    check_bounded("O", a, c, 2 * bound_of(q, kc, vc, sl))


def test_decode_equals_single_row_forward():
    """fa_decode on seqlen n equals fa_fwd (non-causal, Tq = 1) on K[:n]."""
    from exact_tiled_attention_02_amd import fa
    w = inputs.Decode("t", B=3, Hq=8, Hkv=2, Tk_max=700, d=128, seq_lo=1, seq_hi=700, seed=23)
    q, kc, vc, sl = inputs.decode_inputs(w)
    say("fa_decode vs fa_fwd")
    O = run_decode(q, kc, vc, sl, 4)
    bound = bound_of(q, kc, vc, sl)
    for b in range(3):
        n = int(sl[b])
        tq = dev_bf16(q[b:b + 1, :, None, :])
        tk = dev_bf16(np.ascontiguousarray(kc[b:b + 1, :, :n]))
        tv = dev_bf16(np.ascontiguousarray(vc[b:b + 1, :, :n]))
        o = torch.empty(1, 8, 1, 128, dtype=torch.bfloat16, device="cuda")
        fa.fa_fwd(tq, tk, tv, o, None, 1, 8, 2, 1, n, 128, False, 1 / math.sqrt(128))
        torch.cuda.synchronize()
        check_bounded("O", O[b], host_bf16_as_f64(o)[0, :, 0], 2 * bound[b])


def test_automatic_workgroup_count_fills_the_device():
    from exact_tiled_attention_02_amd import fa
    w = inputs.FLASH_DECODE
    n = fa.fa_decode_workgroups(w.B, w.Hq, w.Hkv, w.Tk_max, w.d, 0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say("auto workgroups", n, "CUs", cus)
    assert n >= cus and n % cus == 0


@pytest.mark.parametrize("num_splits", [700, 4096])
def test_decode_many_ranges_per_sequence(num_splits):
    """More than 64 key ranges (workgroups) land on one sequence, so the merge
    combines its partials over several passes; most workgroups of the 4096
    have no keys at all."""
    w = inputs.Decode("t", B=2, Hq=4, Hkv=1, Tk_max=3000, d=128, seq_lo=1, seq_hi=3000, seed=24)
    q, kc, vc, _ = inputs.decode_inputs(w)
    sl = np.array([3000, 1234], np.int32)
    say("fa_decode many ranges", num_splits)
    O = run_decode(q, kc, vc, sl, num_splits)
    Or, _ = oracle.decode_attention(q, kc, vc, sl)
    check_bounded("O", O, Or, bound_of(q, kc, vc, sl))


def test_workspace_reuse_across_shapes():
    """Alternating batch sizes on one stream: the per-segment counters that
    the last range of a segment uses to merge must start from zero whether
    the library's workspace grew, shrank or was reused."""
    cases = [(2, 40), (12, 300), (3, 1000), (12, 300), (2, 40)]
    for i, (B, Tmax) in enumerate(cases):
        w = inputs.Decode("t", B=B, Hq=8, Hkv=2, Tk_max=Tmax, d=128, seq_lo=1, seq_hi=Tmax,
                          seed=30 + i)
        q, kc, vc, sl = inputs.decode_inputs(w)
        say("fa_decode reuse", B, Tmax)
        O = run_decode(q, kc, vc, sl, 0 if i % 2 else 37)
        Or, _ = oracle.decode_attention(q, kc, vc, sl)
        check_bounded("O", O, Or, bound_of(q, kc, vc, sl))


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48, 3 * (1 << 20)])
def test_read_probe_checksum(nbytes):
    """The read probe touches every word exactly once: its XOR checksum
    equals numpy's over the same bytes."""
    from exact_tiled_attention_02_amd import fa
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("fa_read_probe", nbytes)
    fa.fa_read_probe(src, nbytes, sink, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host) if host.size else np.uint32(0)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
