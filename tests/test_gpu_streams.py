"""Calls on two streams at once, from two host threads, through the C ABI:
fa_decode and fa_bwd (the entry points with a library workspace, kept per
(device, stream) and grown on demand) issued concurrently, each thread on its
own stream and growing its workspace at different moments, must give bit for
bit what the same calls give one after another on one stream (every kernel
is deterministic).  Streams are created at the default priority."""
import threading

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


class _Decode:
    def __init__(self, B, Hq, Hkv, Tmax, d, seed):
        w = inputs.Decode("s", B=B, Hq=Hq, Hkv=Hkv, Tk_max=Tmax, d=d, seq_lo=1, seq_hi=Tmax,
                          seed=seed)
        q, kc, vc, sl = inputs.decode_inputs(w)
        self.w = w
        self.q, self.kc, self.vc = dev_bf16(q), dev_bf16(kc), dev_bf16(vc)
        self.sl = torch.from_numpy(np.ascontiguousarray(sl, np.int32)).cuda()
        self.o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")

    def outputs(self):
        return [self.o]

    def issue(self, stream):
        from exact_tiled_attention_02_amd import fa
        w = self.w
        fa.fa_decode(self.q, self.kc, self.vc, self.sl, self.o, w.B, w.Hq, w.Hkv, w.Tk_max, w.d, 0,
                     stream)


class _Backward:
    def __init__(self, Hq, Hkv, T, d, seed):
        from exact_tiled_attention_02_amd import fa
        w = inputs.Prefill("s", B=1, Hq=Hq, Hkv=Hkv, Tq=T, Tk=T, d=d, causal=True, seed=seed)
        q, k, v, do = inputs.prefill_inputs_with_grad(w)
        self.w = w
        self.q, self.k, self.v, self.do = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
        self.o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        fa.fa_fwd(self.q, self.k, self.v, self.o, self.lse, 1, Hq, Hkv, T, T, d, True, w.scale,
                  torch.cuda.current_stream())
        self.dq = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        self.dk = torch.empty(k.shape, dtype=torch.bfloat16, device="cuda")
        self.dv = torch.empty(v.shape, dtype=torch.bfloat16, device="cuda")

    def outputs(self):
        return [self.dq, self.dk, self.dv]

    def issue(self, stream):
        from exact_tiled_attention_02_amd import fa
        w = self.w
        fa.fa_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.dq, self.dk, self.dv,
                  1, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, True, w.scale, stream)


def _bits(jobs):
    return [t.view(torch.int16).cpu().numpy() for j in jobs for t in j.outputs()]


def test_two_streams_from_two_threads_match_one_stream():
    from exact_tiled_attention_02_amd import fa
    fa.fa_release_workspace()
    # Each thread's jobs grow its stream's workspace at a different point:
    # thread 0 goes small -> large, thread 1 large -> small.
    jobs = [
        [_Decode(2, 8, 2, 300, 128, 201), _Backward(4, 2, 200, 64, 202),
         _Decode(16, 32, 8, 3000, 128, 203), _Backward(8, 2, 520, 128, 204)],
        [_Decode(16, 32, 8, 2500, 128, 211), _Backward(8, 4, 600, 128, 212),
         _Decode(3, 8, 2, 200, 64, 213), _Backward(2, 1, 130, 64, 214)],
    ]
    main = torch.cuda.current_stream()
    say("streams: reference on one stream")
    for j in jobs[0] + jobs[1]:
        j.issue(main)
    torch.cuda.synchronize()
    want = [_bits(jobs[0]), _bits(jobs[1])]
    fa.fa_release_workspace()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    errors = []

    def run(i):
        try:
            s = streams[i]
            for _ in range(3):
                for j in jobs[i]:
                    with torch.cuda.stream(s):
                        for t in j.outputs():
                            t.fill_(float("nan"))
                    j.issue(s)
        except Exception as e:   # re-raised on the main thread
            errors.append(e)

    say("streams: two threads, two streams, three rounds each")
    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        got = _bits(jobs[i])
        for n, (a, b) in enumerate(zip(got, want[i])):
            assert np.array_equal(a, b), f"thread {i}, output {n}: differs from the one-stream run"
    fa.fa_release_workspace()
