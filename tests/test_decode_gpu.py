"""GPU parity of lowram_decode_step against the float64 oracle, on seeded
inputs at sizes the oracle finishes in seconds (several blocks and a ragged
tail), with exact stats. Tolerances: relative output error per row 1e-4 for
fp32 activations, 2e-2 for bf16."""
import numpy as np
import pytest
import torch

import synth
from _cases import TOL, gpu_decode, make_case, oracle_decode, rel_err, set_residuals

pytestmark = pytest.mark.gpu

C1 = synth.CONFIGS["c1_tiny_f32"]
C2 = synth.CONFIGS["c2_mistral_group"]
C4 = synth.CONFIGS["c4_llama_262k"]
C5 = synth.CONFIGS["c5_composed"]

SMALL = {
    "f32_ragged": C1.replace(ctx_len=4096 + 37, batch=2),
    "bf16_sel": C2.replace(ctx_len=64 * 40 + 9, batch=2),
    "bf16_r1024_sel": C4.replace(ctx_len=64 * 96 + 50, batch=2, win_cap=64),
    "i8_keep": C5.replace(ctx_len=64 * 48 + 5, batch=3),
    "f32_a_bf16_res": C1.replace(ctx_len=1000, res_dtype="bf16", a_dtype="bf16"),
    "i2_keep": C5.replace(ctx_len=64 * 48 + 5, batch=3, res_dtype="i2"),
    "bf16_i2_sel": C2.replace(ctx_len=64 * 40 + 9, batch=2, res_dtype="i2"),
    "f32_i2": C1.replace(ctx_len=1000, res_dtype="i2"),
}


def check(case, cfg, *, generic, tol=None):
    out, stats = gpu_decode(case, generic=generic)
    ref, rstats = oracle_decode(case)
    err = rel_err(out.float().cpu().numpy(), ref)
    print(f"rel_err={err:.3e}", flush=True)
    assert err <= (tol or TOL[cfg.act]), err
    np.testing.assert_array_equal(stats.cpu().numpy(), rstats)
    return out, stats


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_configs(name, generic):
    cfg = SMALL[name]
    case = make_case(cfg, layer=1, biases=True, win_len=40 if cfg.win_cap else 0)
    check(case, cfg, generic=generic)


@pytest.mark.parametrize("res", ["bf16", "i8"])
@pytest.mark.parametrize("gqa", [1, 2, 3, 8])
def test_gqa_group_sizes(gqa, res):
    """One to eight query heads per KV head. The fused kernel pads the group to
    16 rows in its score, residual and value products; bf16 residual rows take
    the matrix-core path, int8 rows the per-row one."""
    base = C2 if res == "bf16" else C5
    cfg = base.replace(ctx_len=64 * 24 + 11, batch=2, n_kv_heads=2, n_q_heads=2 * gqa)
    case = make_case(cfg, layer=1, biases=True)
    check(case, cfg, generic=False)


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
def test_peaked_attention(generic):
    """Query rescaled so logits have a spread of about 4: a score-path bug
    cannot hide behind a near-uniform softmax."""
    cfg = SMALL["bf16_sel"]
    case = make_case(cfg, layer=2, q_scale=180.0)
    check(case, cfg, generic=generic)
    cfg = SMALL["f32_ragged"]
    case = make_case(cfg, layer=2, q_scale=180.0)
    check(case, cfg, generic=generic)


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
def test_no_residuals_and_every_token_a_residual(generic):
    for cfg in (SMALL["f32_ragged"], SMALL["bf16_sel"], SMALL["i8_keep"], SMALL["i2_keep"]):
        case = make_case(cfg, layer=0)
        bsz = case["q"].shape[0]
        set_residuals(case, cfg, torch.zeros(bsz, 8, 0, dtype=torch.int32))
        check(case, cfg, generic=generic)
        set_residuals(case, cfg, torch.arange(cfg.ctx_len, dtype=torch.int32).expand(bsz, 8, -1))
        check(case, cfg, generic=generic)


@pytest.mark.parametrize("res", ["bf16", "i8", "i2"])
def test_residual_rows_per_block_around_batch_sizes(res):
    """Blocks holding 1, 15, 16, 17, 33 and 64 residual rows, every block
    attended: the fused kernel sums bf16 rows 16 at a time, int8 rows 32 at a
    time and 2-bit rows 64 at a time (two steps of 32) on the matrix cores."""
    base = C2 if res == "bf16" else C5
    cfg = base.replace(ctx_len=64 * 8, batch=2, sel_den=1, evict_half=False, res_dtype=res)
    case = make_case(cfg, layer=0)
    rows = []
    for blk, n in enumerate([1, 15, 16, 17, 33, 64, 0, 2]):
        rows += list(range(blk * 64 + (64 - n) // 2, blk * 64 + (64 - n) // 2 + n))
    idx = torch.tensor(rows, dtype=torch.int32).expand(2, 8, -1)
    set_residuals(case, cfg, idx)
    check(case, cfg, generic=False)


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
@pytest.mark.parametrize("name", ["i2_keep", "f32_i2", "i8_keep"])
def test_quantised_residuals_carry_the_output(name, generic):
    """Every token holds a 2-bit or int8 residual of about the values' size,
    so the output moves by far more than the tolerance if a code is decoded
    from the wrong bits or row, with the wrong level offset or without its
    scale."""
    cfg = SMALL[name]
    case = make_case(cfg, layer=7)
    bsz = case["q"].shape[0]
    set_residuals(case, cfg, torch.arange(cfg.ctx_len, dtype=torch.int32).expand(bsz, 8, -1))
    case["res_scale"] = case["res_scale"] * 20.0
    ref, _ = oracle_decode(case)
    plain = dict(case, res_scale=torch.zeros_like(case["res_scale"]))
    ref0, _ = oracle_decode(plain)
    assert rel_err(ref0, ref) > 10 * TOL[cfg.act]
    check(case, cfg, generic=generic)


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
def test_single_block_all_blocks_last_partial_block(generic):
    cfg = SMALL["bf16_sel"]
    nb = cfg.nb
    case = make_case(cfg, layer=3)
    for sel in ([[nb - 1], [0]], [[5], [nb - 1]], [list(range(nb))] * 2):
        case["sel"] = torch.tensor(sel, dtype=torch.int32)
        check(case, cfg, generic=generic)
    case["sel"] = None
    check(case, cfg, generic=generic)


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
@pytest.mark.parametrize("with_keep", [False, True], ids=["direct", "compacted"])
def test_ragged_selection_rows_padded(generic, with_keep):
    """Rows of one batch that select different numbers of blocks, padded with
    -1 and with an out-of-range index; one row is padding only."""
    cfg = SMALL["bf16_sel"].replace(batch=3)
    nb = cfg.nb
    case = make_case(cfg, layer=7)
    case["sel"] = torch.tensor([[0, 3, 7, nb - 1, -1, -1],
                                [-1, -1, -1, -1, -1, -1],
                                [2, 5, nb, -1, 9, -7]], dtype=torch.int32)
    case["keep"] = torch.ones(3, nb, dtype=torch.uint8) if with_keep else None
    case["win_len"] = 0
    out, stats = check(case, cfg, generic=generic)
    assert not out[1].float().abs().sum().item() and stats[1].abs().sum().item() == 0


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
def test_window_lengths(generic):
    cfg = SMALL["bf16_r1024_sel"]
    case = make_case(cfg, layer=4)
    for w in (0, 1, 63, 64):
        case["win_len"] = w
        check(case, cfg, generic=generic)


@pytest.mark.parametrize("name,act_cfg", [("bf16", C4.replace(ctx_len=64 * 20 + 3, batch=2, win_cap=1024)),
                                          ("f32", C1.replace(ctx_len=64 * 12 + 5, batch=2, win_cap=1024))])
def test_long_windows(name, act_cfg):
    """Windows that cross the combine's 128-token batches (eight waves of 16
    tokens each, later batches loaded and folded in turn), up to the full
    1024-token capacity; dominant window scores (query scaled up) so that an
    unmerged or misscaled batch shows in the output."""
    case = make_case(act_cfg, layer=2, q_scale=4.0)
    for w in (127, 128, 129, 300, 1024):
        case["win_len"] = w
        check(case, act_cfg, generic=False)


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
def test_window_only_sequence(generic):
    """Sequence 1 has every block evicted but 40 window tokens: the combine
    has no partial record for it (and must not read a stale one) and attends
    the window alone; sequence 0 keeps its blocks."""
    cfg = SMALL["bf16_r1024_sel"]
    case = make_case(cfg, layer=3)
    nb = -(-cfg.ctx_len // 64)
    case["keep"] = torch.ones(2, nb, dtype=torch.uint8)
    case["keep"][1] = 0
    case["win_len"] = 40
    out, stats = check(case, cfg, generic=generic)
    assert stats[1, :, 1].abs().sum().item() == 0 and (stats[1, :, 0] == 40).all()


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
def test_sequence_with_everything_evicted(generic):
    cfg = SMALL["i8_keep"]
    case = make_case(cfg, layer=5)
    case["keep"][1] = 0
    out, stats = check(case, cfg, generic=generic)
    assert not out[1].float().abs().sum().item()
    assert stats[1].abs().sum().item() == 0


@pytest.mark.parametrize("generic", [True, False], ids=["generic", "auto"])
def test_bitwise_rerun(generic):
    cfg = SMALL["bf16_sel"]
    case = make_case(cfg, layer=6)
    o1, s1 = gpu_decode(case, generic=generic)
    o2, s2 = gpu_decode(case, generic=generic)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_c1_full_config_four_layers():
    """The tiny fp32 workload as configured: batch 1, T=4096, one group of 4
    layers, r=256, h=64, every block, k=819."""
    for layer in range(C1.n_layers):
        case = make_case(C1, layer=layer, biases=False)
        check(case, C1, generic=False)


@pytest.mark.parametrize("seed", range(8))
def test_randomised_shapes_and_encodings(seed):
    """Seeded draws over the step's options, several at once: A bf16 or int8;
    residuals bf16, int8 or 2-bit at 0-50% of the tokens; 1, 2 or 4 KV heads
    with 1-8 query heads each; ragged context; rank 64-512; hidden 64-256;
    every block or a selection; eviction flags; a window. Seeds 6 and 7 force
    the fp32 SIMT kernel on the same kind of draw."""
    rng = np.random.default_rng(1000 + seed)
    hkv = int(rng.choice([1, 2, 4]))
    win_cap = int(rng.choice([0, 64]))
    cfg = C2.replace(ctx_len=int(rng.integers(64 * 6, 64 * 40)), batch=int(rng.integers(1, 4)),
                     n_kv_heads=hkv, n_q_heads=hkv * int(rng.choice([1, 2, 3, 4, 8])),
                     rank=int(rng.choice([64, 128, 256, 512])), mlp_hidden=int(rng.choice([64, 128, 256])),
                     sel_den=int(rng.choice([1, 2, 4])), evict_half=bool(rng.integers(0, 2)),
                     a_dtype=str(rng.choice(["bf16", "i8"])), res_dtype=str(rng.choice(["bf16", "i8", "i2"])),
                     res_frac=(int(rng.integers(0, 6)), 10), win_cap=win_cap, seed=seed)
    print(cfg, flush=True)
    case = make_case(cfg, layer=int(rng.integers(0, 4)),
                     win_len=int(rng.integers(1, win_cap + 1)) if win_cap else 0)
    check(case, cfg, generic=seed >= 6)
