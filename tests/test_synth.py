"""The seeded input generator: determinism and the structural rules of the
selection, eviction and residual sets (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
import synth


def small(cfg_name, **kw):
    return synth.CONFIGS[cfg_name].replace(**kw)


def test_residual_counts_per_config():
    want = {"c1_tiny_f32": 819, "c2_mistral_group": 6553, "c3_llama_131k": 26214,
            "c4_llama_262k": 52428, "c5_composed": 13107}
    for name, k in want.items():
        assert synth.CONFIGS[name].n_res == k
    assert synth.RANK_C5.n_res == 13107


def test_layer_inputs_are_deterministic():
    cfg = small("c2_mistral_group", ctx_len=1000, rank=64, mlp_hidden=32)
    x = synth.gen_layer(cfg, 1, "cpu", biases=True)
    y = synth.gen_layer(cfg, 1, "cpu", biases=True)
    for k in x:
        if x[k] is None:
            assert y[k] is None
        else:
            assert torch.equal(x[k], y[k]), k
    z = synth.gen_layer(cfg, 2, "cpu", biases=True)
    assert not torch.equal(x["q"], z["q"])
    assert x["q"].dtype == torch.bfloat16 and x["bl"].shape == (1, 8 * 128, 64)


def test_selection_rules():
    cfg = small("c3_llama_131k", ctx_len=64 * 96, batch=3)      # nb = 96, n_sel = 12
    sel = synth.gen_layer(cfg, 0, "cpu")["sel"]
    assert sel.shape == (3, 12) and sel.dtype == torch.int32
    for row in sel.tolist():
        assert row == sorted(set(row))
        assert {0, 1, 94, 95} <= set(row)
        assert all(0 <= i < 96 for i in row)


def test_eviction_rules():
    cfg = small("c5_composed", ctx_len=64 * 40, batch=2)
    keep = synth.gen_layer(cfg, 3, "cpu")["keep"]
    assert keep.shape == (2, 40)
    for row in keep.tolist():
        assert row.count(0) == 20
        assert row[0] == row[1] == row[38] == row[39] == 1


def test_residual_sets_and_block_ptr_match_the_oracle_definition():
    cfg = small("c2_mistral_group", ctx_len=64 * 10 + 13, rank=64, mlp_hidden=32, batch=2)
    x = synth.gen_layer(cfg, 0, "cpu")
    idx, ptr = x["res_idx"], x["res_ptr"]
    assert idx.shape == (2, 8, cfg.n_res)
    for b in range(2):
        for h in range(8):
            row = idx[b, h].tolist()
            assert row == sorted(set(row)) and 0 <= row[0] and row[-1] < cfg.ctx_len
            np.testing.assert_array_equal(ptr[b, h].numpy(), oracle.block_ptr(row, cfg.ctx_len, 64))


def test_int8_inputs():
    cfg = small("c5_composed", ctx_len=256, batch=1)
    a, s = synth.gen_group_factor(cfg, 0, "cpu")
    assert a.dtype == torch.int8 and s.shape == (1, 256) and s.dtype == torch.float32
    assert int(a.abs().max()) <= 127
    x = synth.gen_layer(cfg, 0, "cpu")
    assert x["res_val"].dtype == torch.int8 and x["res_scale"].shape == (1, 8, cfg.n_res)


def test_rank_inputs_plant_a_tie_group_across_the_kth_place():
    rc = synth.RankConfig(1, 3000, n_kv_heads=2, res_frac=(1, 10), in_dtype="bf16")
    v, vh = synth.gen_rank_inputs(rc, "cpu")
    vf = v.float().numpy()
    hf = vh.float().numpy()
    k = rc.n_res
    for h in range(2):
        e = oracle.residual_error(vf[0, :, h], hf[0, :, h])
        order = np.sort(e)[::-1]
        kth = order[k - 1]
        assert order[k] == kth                       # the k-th value is tied with the next
        assert np.count_nonzero(e == kth) >= 2
