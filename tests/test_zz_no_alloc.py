"""lowram_decode_step_noalloc, the decode step for callers that cannot
allocate: its scratch is the library's static device array instead of a
caller workspace. Called through the C ABI, its outputs and stats must equal
those of lowram_decode_step on the same inputs bit for bit (same kernels,
same order of operations), on two calls in a row, the second with a smaller
input, and agree with the float64 oracle; shapes that need more scratch than
the array holds are refused before any HIP call."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from _cases import TOL, make_case, oracle_decode, rel_err, to
import long_context_decode_lowram_amd as L

pytestmark = pytest.mark.gpu


def _args(case):
    c = to(case, "cuda")
    out = torch.full(c["q"].shape, float("nan"), dtype=c["q"].dtype, device="cuda")
    stats = torch.full((c["q"].shape[0], c["bl"].shape[1] // 128, 2), -7, dtype=torch.int32, device="cuda")
    args = L.make_decode_args(c["q"], c["a"], c["bl"], c["w_lin"], c["w1"], c["w2"], c["res_idx"], c["res_val"],
                              c["res_ptr"], out, a_scale=c["a_scale"], b1=c["b1"], b2=c["b2"],
                              res_scale=c["res_scale"], sel=c["sel"], keep=c["keep"], win_k=c["win_k"],
                              win_v=c["win_v"], win_len=c["win_len"], stats=stats)
    return c, args, out, stats


def _with_workspace(case):
    c, args, out, stats = _args(case)
    ws = torch.empty(L.decode_workspace_size(args), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    L.decode_launch(args)
    torch.cuda.synchronize()
    return out, stats


def _no_alloc(case):
    c, args, out, stats = _args(case)
    assert L.decode_workspace_size(args) <= L.NOALLOC_SCRATCH_BYTES
    args.workspace, args.workspace_bytes = None, 0          # ignored by this entry point
    L.decode_launch_noalloc(args)
    torch.cuda.synchronize()
    return out, stats


def test_no_alloc_matches_the_workspace_entry_point_two_calls():
    big = synth.CONFIGS["c4_llama_262k"].replace(ctx_len=64 * 600 + 21, batch=3, win_cap=64)
    small = synth.CONFIGS["c2_mistral_group"].replace(ctx_len=64 * 40 + 9, batch=2)
    cases = [(big, make_case(big, layer=3, biases=True, win_len=40)), (small, make_case(small, layer=1))]
    refs = [_with_workspace(c) for _, c in cases]
    for (cfg, case), (ref_out, ref_stats) in zip(cases, refs):
        out, stats = _no_alloc(case)
        assert torch.equal(out, ref_out)
        assert torch.equal(stats, ref_stats)
        oref, ostats = oracle_decode(case)
        err = rel_err(out.float().cpu().numpy(), oref)
        print(f"{cfg.name} B={cfg.batch} T={cfg.ctx_len}: rel_err={err:.2e}", flush=True)
        assert err <= TOL[cfg.act]
        np.testing.assert_array_equal(stats.cpu().numpy(), ostats)


def test_no_alloc_int8_with_eviction_flags_after_a_larger_call():
    cfg = synth.CONFIGS["c5_composed"].replace(ctx_len=64 * 48 + 5, batch=3)
    big = synth.CONFIGS["c4_llama_262k"].replace(ctx_len=64 * 900, batch=4, win_cap=0)
    _no_alloc(make_case(big, layer=0))                       # leaves its records in the shared array
    case = make_case(cfg, layer=2)
    ref_out, ref_stats = _with_workspace(case)
    out, stats = _no_alloc(case)
    assert torch.equal(out, ref_out) and torch.equal(stats, ref_stats)


def test_no_alloc_refuses_shapes_beyond_the_array():
    """Composed-workload shapes (batch 12, every one of 2048 blocks a
    candidate) need more scratch than the array: refused on the host."""
    a = L.DecodeArgs()
    a.batch, a.ctx_len, a.n_q_heads, a.n_kv_heads, a.head_dim = 12, 131072, 32, 8, 128
    a.rank, a.mlp_hidden, a.block_size, a.n_res = 512, 256, 64, 13107
    a.act_dtype, a.a_dtype, a.res_dtype = L.BF16, L.I8, L.I8
    for n in ("q", "a", "a_scale", "b_l", "w_lin", "w1", "w2", "res_idx", "res_val", "res_scale", "res_blk_ptr",
              "keep", "out"):
        setattr(a, n, 0x100000)
    assert L.decode_workspace_size(a) > L.NOALLOC_SCRATCH_BYTES
    rc = L.lib().lowram_decode_step_noalloc(ctypes.byref(a), None)
    assert rc == L._binding.ERR_WORKSPACE
    assert "scratch" in L.last_error()
