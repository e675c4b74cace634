"""lowram_decode_step under stream capture. The entry point only enqueues
kernels (no allocation, no synchronisation, no memset), so a HIP graph can
hold a whole step of layer calls. The graph is replayed several times with
eager work and synchronisations between the replays, the outputs cleared
before each replay, and every replay must give the eager outputs bit for
bit (the kernels are deterministic)."""
import pytest
import torch

import synth
from _cases import make_case, oracle_decode, rel_err, TOL, to
import long_context_decode_lowram_amd as L

pytestmark = pytest.mark.gpu

C2 = synth.CONFIGS["c2_mistral_group"]
C5 = synth.CONFIGS["c5_composed"]


def _calls(cfgs):
    cases, calls, outs, stats = [], [], [], []
    for layer, cfg in enumerate(cfgs):
        c = to(make_case(cfg, layer=layer), "cuda")
        out = torch.empty(c["q"].shape, dtype=c["q"].dtype, device="cuda")
        st = torch.empty(c["q"].shape[0], c["bl"].shape[1] // 128, 2, dtype=torch.int32, device="cuda")
        args = L.make_decode_args(c["q"], c["a"], c["bl"], c["w_lin"], c["w1"], c["w2"], c["res_idx"],
                                  c["res_val"], c["res_ptr"], out, a_scale=c["a_scale"], b1=c["b1"],
                                  b2=c["b2"], res_scale=c["res_scale"], sel=c["sel"], keep=c["keep"],
                                  win_k=c["win_k"], win_v=c["win_v"], win_len=c["win_len"], stats=st)
        cases.append(c)
        calls.append(args)
        outs.append(out)
        stats.append(st)
    ws_bytes = max(L.decode_workspace_size(a) for a in calls)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    for a in calls:
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws_bytes
    return cases, calls, outs, stats, ws


def test_graph_of_layer_calls_replays_the_eager_results():
    # bf16 with a selection, and int8 A / int8 residuals with eviction flags
    # (the compaction pass runs too), as consecutive layer calls.
    cfgs = [C2.replace(ctx_len=64 * 40 + 9, batch=2), C5.replace(ctx_len=64 * 48 + 5, batch=3),
            C2.replace(ctx_len=64 * 40 + 9, batch=2, res_dtype="i2")]
    cases, calls, outs, stats, ws = _calls(cfgs)

    for a in calls:
        L.decode_launch(a)
    torch.cuda.synchronize()
    eager = [(o.clone(), s.clone()) for o, s in zip(outs, stats)]
    for c, (o, s), cfg in zip(cases, eager, cfgs):
        ref, rstats = oracle_decode(c)
        assert rel_err(o.float().cpu().numpy(), ref) <= TOL[cfg.act]
        assert (s.cpu().numpy() == rstats).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for a in calls:
            L.decode_launch(a, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for a in calls:
            L.decode_launch(a, torch.cuda.current_stream())
    torch.cuda.synchronize()

    other_cases, other_calls, other_outs, _, _ = _calls([C2.replace(ctx_len=64 * 12 + 3, batch=1, seed=5)])
    for rep in range(4):
        for o, s in zip(outs, stats):
            o.fill_(float("nan"))
            s.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        # eager work of the program's own between replays
        L.decode_launch(other_calls[0])
        x = torch.randn(1 << 20, device="cuda")
        _ = (x * 2).sum()
        torch.cuda.synchronize()
        for (o, s), (eo, es) in zip(zip(outs, stats), eager):
            assert torch.equal(o, eo), f"replay {rep}: output differs"
            assert torch.equal(s, es), f"replay {rep}: stats differ"


class _Ev:
    """Ordering-only hipEvent_t handles and stream waits through the HIP runtime."""

    def __init__(self):
        import ctypes
        self.c = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]

    def create(self):
        e = self.c.c_void_p()
        assert self.lib.hipEventCreateWithFlags(self.c.byref(e), 2) == 0
        return e.value

    def record(self, e, stream):
        assert self.lib.hipEventRecord(self.c.c_void_p(e), self.c.c_void_p(stream.cuda_stream)) == 0

    def wait(self, stream, e):
        assert self.lib.hipStreamWaitEvent(self.c.c_void_p(stream.cuda_stream), self.c.c_void_p(e), 0) == 0


def test_combine_on_a_second_stream_overlapping_the_next_call():
    """Layer calls with the combine on a second stream and two workspaces
    used in turn (call l+2 waits for call l's combine), eagerly and as a
    graph replayed between eager work, give the single-stream outputs bit for
    bit."""
    cfgs = [C2.replace(ctx_len=64 * 40 + 9, batch=2, seed=s) for s in range(3)] + \
           [C5.replace(ctx_len=64 * 48 + 5, batch=3), C2.replace(ctx_len=64 * 40 + 9, batch=2, res_dtype="i2")]
    cases, calls, outs, stats, ws = _calls(cfgs)
    for a in calls:
        L.decode_launch(a)
    torch.cuda.synchronize()
    eager = [(o.clone(), s.clone()) for o, s in zip(outs, stats)]

    ev = _Ev()
    ws2 = torch.empty_like(ws)
    cs = torch.cuda.Stream()
    ready = [ev.create() for _ in calls]
    done = [ev.create() for _ in calls]
    for l, a in enumerate(calls):
        a.workspace = (ws if l % 2 == 0 else ws2).data_ptr()
        a.combine_stream, a.combine_ready = cs.cuda_stream, ready[l]

    def step(main):
        for l, a in enumerate(calls):
            if l >= 2:
                ev.wait(main, done[l - 2])
            L.decode_launch(a, main)
            ev.record(done[l], cs)
        for l in range(len(calls) - 2, len(calls)):
            ev.wait(main, done[l])

    def clear():
        for o, s in zip(outs, stats):
            o.fill_(float("nan"))
            s.fill_(-9)
        torch.cuda.synchronize()

    def check(what):
        for (o, s), (eo, es) in zip(zip(outs, stats), eager):
            assert torch.equal(o, eo), f"{what}: output differs"
            assert torch.equal(s, es), f"{what}: stats differ"

    clear()
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    check("eager, two streams")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        clear()
        g.replay()
        x = torch.randn(1 << 20, device="cuda")
        _ = (x * 2).sum()
        torch.cuda.synchronize()
        check(f"replay {rep}")
