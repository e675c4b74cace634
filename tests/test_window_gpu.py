"""The recent window as the long-context protocol runs it: each decode step
appends the new token's exact key and value to every layer's window buffer
(lowram_window_append), and the decode calls read the window length from the
device count that the append advanced, so one captured graph serves every
step (explainer, prefill/decode paragraph: new tokens kept exactly). Also the
validate mode's defect bits on malformed index data. Parity against the
float64 oracle; graph replays against eager runs bit for bit."""
import numpy as np
import pytest
import torch

import synth
from _cases import TOL, WindowSession as Session, make_case, oracle_decode, rel_err, to
import long_context_decode_lowram_amd as L

pytestmark = pytest.mark.gpu

C2 = synth.CONFIGS["c2_mistral_group"]
C4 = synth.CONFIGS["c4_llama_262k"]


def test_appended_window_every_step_against_the_oracle():
    cfg = C4.replace(ctx_len=64 * 80 + 5, batch=2, n_layers=2)          # nb 81, 5 blocks selected
    s = Session(cfg, cap=16)
    appended_k = []
    for step in range(6):
        st = s.stage(step)
        appended_k.append(st["new_k"].clone())
        s.launch()
        torch.cuda.synchronize()
        assert s.count.tolist() == [step + 1] * cfg.n_layers
        # the window holds exactly the tokens appended so far, in order
        assert torch.equal(s.win_k[:, :, step], st["new_k"]) and torch.equal(s.win_v[:, :, step], st["new_v"])
        for l in range(cfg.n_layers):
            ref, rstats = s.oracle(l, step + 1, st)
            err = rel_err(s.outs[l].float().cpu().numpy(), ref)
            print(f"step {step} layer {l}: rel_err={err:.2e}", flush=True)
            assert err <= TOL[cfg.act]
            np.testing.assert_array_equal(s.stats[l].cpu().numpy(), rstats)
    assert torch.equal(s.win_k[:, :, :6].permute(2, 0, 1, 3), torch.stack(appended_k))


def test_graph_of_append_and_layer_calls_replays_the_eager_steps():
    cfg = C4.replace(ctx_len=64 * 80 + 5, batch=2, n_layers=3)
    s = Session(cfg, cap=4)                                          # fills up at step 4
    eager = []
    for step in range(6):
        s.stage(step)
        s.launch()
        torch.cuda.synchronize()
        eager.append([(o.clone(), t.clone()) for o, t in zip(s.outs, s.stats)])
    assert s.count.tolist() == [4] * cfg.n_layers                   # a full buffer keeps its count
    # The last step attended the four first appended tokens.
    st = synth.gen_step_inputs(cfg, 5, "cuda")
    for l in range(cfg.n_layers):
        ref, rstats = s.oracle(l, 4, st)
        assert rel_err(eager[5][l][0].float().cpu().numpy(), ref) <= TOL[cfg.act]
        np.testing.assert_array_equal(eager[5][l][1].cpu().numpy(), rstats)

    s.count.zero_()
    s.win_k.zero_()
    s.win_v.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s.launch(side)                                               # warm the launch path off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    s.count.zero_()
    s.win_k.zero_()
    s.win_v.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s.launch(torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert s.count.tolist() == [0] * cfg.n_layers                    # capture ran nothing
    for step in range(6):
        s.stage(step)
        for o in s.outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        x = torch.randn(1 << 20, device="cuda")                       # the program's own work between replays
        torch.cuda.synchronize()
        assert float(x.abs().sum()) > 0
        for l in range(cfg.n_layers):
            assert torch.equal(s.outs[l], eager[step][l][0]), (step, l)
            assert torch.equal(s.stats[l], eager[step][l][1]), (step, l)
    assert s.count.tolist() == [4] * cfg.n_layers


# ------------------------------------------------------------ validate mode
def _validated(case, flags, *, generic=False, win_len_dev=None, win_len=None):
    c = to(case, "cuda")
    out = torch.empty_like(c["q"])
    stats = torch.empty(c["q"].shape[0], c["bl"].shape[1] // 128, 2, dtype=torch.int32, device="cuda")
    flags.zero_()
    args = L.make_decode_args(c["q"], c["a"], c["bl"], c["w_lin"], c["w1"], c["w2"], c["res_idx"], c["res_val"],
                              c["res_ptr"], out, a_scale=c["a_scale"], b1=c["b1"], b2=c["b2"],
                              res_scale=c["res_scale"], sel=c["sel"], keep=c["keep"], win_k=c["win_k"],
                              win_v=c["win_v"], win_len=c["win_len"] if win_len is None else win_len, stats=stats,
                              generic=generic, validate=flags, win_len_dev=win_len_dev)
    ws = torch.empty(L.decode_workspace_size(args), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    L.decode_launch(args)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    return int(flags.item()), out, stats


@pytest.mark.parametrize("generic", [False, True], ids=["auto", "generic"])
def test_validate_mode_names_each_defect(generic):
    cfg = C4.replace(ctx_len=64 * 96 + 50, batch=2, win_cap=64)     # nb 97, 6 blocks selected, a window
    base = make_case(cfg, layer=2, biases=True, win_len=20)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    bits, out, stats = _validated(base, flags, generic=generic)
    assert bits == 0
    ref, rstats = oracle_decode(base)
    assert rel_err(out.float().cpu().numpy(), ref) <= TOL[cfg.act]
    np.testing.assert_array_equal(stats.cpu().numpy(), rstats)

    def mutated(**kw):
        c = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in base.items()}
        c.update(kw)
        return c

    sel = base["sel"].clone()
    sel[0, 2] = sel[0, 1]                                           # duplicate entry
    assert _validated(mutated(sel=sel), flags, generic=generic)[0] & L.CHECK_SEL_ORDER
    sel = base["sel"].flip(1).contiguous()                          # descending
    assert _validated(mutated(sel=sel), flags, generic=generic)[0] & L.CHECK_SEL_ORDER
    sel = base["sel"].clone()
    sel[1, 0], sel[1, -1] = -1, cfg.nb + 3                           # padding only: still valid
    assert _validated(mutated(sel=sel), flags, generic=generic)[0] == 0
    idx = base["res_idx"].clone()
    idx[1, 3, -1] = cfg.ctx_len                                      # past the cache
    assert _validated(mutated(res_idx=idx), flags, generic=generic)[0] & L.CHECK_RES_RANGE
    idx = base["res_idx"].clone()
    i0 = int(torch.nonzero(idx[0, 0, 1:] // 64 == idx[0, 0, :-1] // 64)[0])   # two slots in one block
    idx[0, 0, i0], idx[0, 0, i0 + 1] = idx[0, 0, i0 + 1].item(), idx[0, 0, i0].item()
    bits = _validated(mutated(res_idx=idx), flags, generic=generic)[0]
    assert bits & L.CHECK_RES_ORDER and not bits & L.CHECK_RES_PTR
    ptr = base["res_ptr"].clone()
    ptr[0, 5, 7] += 1                                                # one block pointer off by one
    assert _validated(mutated(res_ptr=ptr), flags, generic=generic)[0] == L.CHECK_RES_PTR
    ptr = base["res_ptr"].clone()
    ptr[1, 2, -1] = 10 ** 6                                          # far past n_res
    assert _validated(mutated(res_ptr=ptr), flags, generic=generic)[0] & L.CHECK_RES_PTR
    # A device window count beyond its bound is flagged and clamped to it.
    cnt = torch.tensor([base["win_len"] + 7], dtype=torch.int32, device="cuda")
    bits, out, stats = _validated(base, flags, generic=generic, win_len_dev=cnt)
    assert bits == L.CHECK_WIN_LEN
    assert rel_err(out.float().cpu().numpy(), ref) <= TOL[cfg.act]
    cnt.fill_(5)
    bits, out, stats = _validated(base, flags, generic=generic, win_len_dev=cnt)
    assert bits == 0
    ref5, rstats5 = oracle_decode(dict(base, win_len=5))
    assert rel_err(out.float().cpu().numpy(), ref5) <= TOL[cfg.act]
    np.testing.assert_array_equal(stats.cpu().numpy(), rstats5)


def test_validate_mode_with_eviction_flags_and_int8():
    cfg = synth.CONFIGS["c5_composed"].replace(ctx_len=64 * 48 + 5, batch=3)
    base = make_case(cfg, layer=1)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert _validated(base, flags)[0] == 0
    idx = base["res_idx"].clone()
    idx[2, 1, 0] = -5
    assert _validated(dict(base, res_idx=idx), flags)[0] & L.CHECK_RES_RANGE
