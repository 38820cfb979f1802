"""HIP-graph capture of the entry points that neither allocate nor enqueue
memsets (fa_fwd, fa_fwd_fp8, fa_decode_noalloc), through the C ABI and
torch.cuda.CUDAGraph: one graph holds a bf16 forward, an 8-bit forward and a
decode.  It is replayed several times, with the program's own eager work,
output clearing and synchronisation between replays, and every replay must
reproduce the eager calls bit for bit (the kernels are deterministic); new
data copied into the captured input buffers must give what eager calls give
on that data, so the graph reads its inputs at replay time."""
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


def _host_data(seed):
    """Inputs of the three calls for one seed, as host arrays."""
    wf = inputs.Prefill("g", B=1, Hq=8, Hkv=2, Tq=300, Tk=300, d=128, causal=True, seed=seed)
    w8 = inputs.Prefill("g8", B=1, Hq=4, Hkv=2, Tq=200, Tk=200, d=64, causal=True, seed=seed + 1)
    wd = inputs.Decode("gd", B=4, Hq=8, Hkv=2, Tk_max=700, d=128, seq_lo=1, seq_hi=700,
                       seed=seed + 2)
    return (wf, inputs.prefill_inputs(wf)), (w8, inputs.prefill_inputs_fp8(w8)), \
        (wd, inputs.decode_inputs(wd))


class _Calls:
    """Device buffers of the three calls; `issue` enqueues them on a stream."""

    def __init__(self, host):
        (wf, (q, k, v)), (w8, fp8), (wd, (dq, kc, vc, sl)) = host
        self.wf, self.w8, self.wd = wf, w8, wd
        self.q, self.k, self.v = dev_bf16(q), dev_bf16(k), dev_bf16(v)
        self.o = torch.empty((wf.B, wf.Hq, wf.Tq, wf.d), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((wf.B, wf.Hq, wf.Tq), dtype=torch.float32, device="cuda")
        q8, k8, v8, qs, ks, vs = fp8
        self.c8 = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q8, k8, v8)]
        self.s8 = [torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda() for x in (qs, ks, vs)]
        self.o8 = torch.empty((w8.B, w8.Hq, w8.Tq, w8.d), dtype=torch.bfloat16, device="cuda")
        self.lse8 = torch.empty((w8.B, w8.Hq, w8.Tq), dtype=torch.float32, device="cuda")
        self.dq, self.kc, self.vc = dev_bf16(dq), dev_bf16(kc), dev_bf16(vc)
        self.sl = torch.from_numpy(np.ascontiguousarray(sl, np.int32)).cuda()
        self.od = torch.empty((wd.B, wd.Hq, wd.d), dtype=torch.bfloat16, device="cuda")

    def load(self, other):
        """Copy another data set's inputs into these (captured) buffers."""
        for a, b in ((self.q, other.q), (self.k, other.k), (self.v, other.v), (self.dq, other.dq),
                     (self.kc, other.kc), (self.vc, other.vc), (self.sl, other.sl)):
            a.copy_(b)
        for a, b in zip(self.c8 + self.s8, other.c8 + other.s8):
            a.copy_(b)

    def clear(self):
        for t in self.outputs():
            t.fill_(float("nan"))

    def outputs(self):
        return [self.o, self.lse, self.o8, self.lse8, self.od]

    def issue(self, stream):
        from exact_tiled_attention_02_amd import fa
        wf, w8, wd = self.wf, self.w8, self.wd
        fa.fa_fwd(self.q, self.k, self.v, self.o, self.lse, wf.B, wf.Hq, wf.Hkv, wf.Tq, wf.Tk,
                  wf.d, True, wf.scale, stream)
        fa.fa_fwd_fp8(*self.c8, *self.s8, self.o8, self.lse8, w8.B, w8.Hq, w8.Hkv, w8.Tq, w8.Tk,
                      w8.d, True, w8.scale, stream)
        fa.fa_decode_noalloc(self.dq, self.kc, self.vc, self.sl, self.od, wd.B, wd.Hq, wd.Hkv,
                             wd.Tk_max, wd.d, 0, stream)


def _bits(ts):
    return [t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
            for t in ts]


def _same(got, want, what):
    for name, a, b in zip(("o", "lse", "o fp8", "lse fp8", "o decode"), got, want):
        assert np.array_equal(a, b), f"{what}: {name} differs from the eager call"


def test_graph_replays_match_eager_calls():
    captured = _Calls(_host_data(81))
    other = _Calls(_host_data(91))        # second data set, and eager work between replays
    stream = torch.cuda.current_stream()

    # Eager reference on both data sets (also the first fa_decode_noalloc call
    # on this device, which looks up its workspace before any capture).
    say("graph: eager calls")
    captured.issue(stream)
    other.issue(stream)
    torch.cuda.synchronize()
    want_a, want_b = _bits(captured.outputs()), _bits(other.outputs())

    say("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured.issue(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(3):
        say("graph: replay", rep)
        captured.clear()
        other.clear()
        other.issue(stream)               # eager work of the program between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(_bits(captured.outputs()), want_a, f"replay {rep}")
        _same(_bits(other.outputs()), want_b, f"eager call beside replay {rep}")

    say("graph: replay on new inputs")
    captured.load(other)
    captured.clear()
    g.replay()
    torch.cuda.synchronize()
    _same(_bits(captured.outputs()), want_b, "replay on the second data set")
