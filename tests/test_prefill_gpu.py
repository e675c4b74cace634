"""GPU parity of the fused prefill ranking (lowram_prefill_rank) against the
float64 oracle.

V_hat is computed in the library with bf16 MFMA products, so it matches the
oracle's float64 V_hat within the bf16 tolerance; the ranking is a discrete
function of V_hat, so it is checked exactly against the oracle's ranking of
the true values V against the V_hat the library returns (its fp32 copy):
errors bit-equal, index sets and block pointers equal, residuals equal to the
oracle's encoding of V - V_hat. That also shows the second pass, which
recomputes V_hat for the chosen tokens, reproduced the ranked V_hat bit for bit.
"""
import numpy as np
import pytest
import torch

import long_context_decode_lowram_amd as L
import oracle
import synth

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _np(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


def _launch(pc, res_dtype):
    x = synth.gen_prefill_inputs(pc, "cuda")
    out = L.prefill_rank(x["a"], x["b_l"], x["w_lin"], x["w1"], x["w2"], x["v"], pc.n_res, res_dtype,
                         group=pc.group, b1=x["b1"], b2=x["b2"], want_err=True, want_v_hat=True)
    torch.cuda.synchronize()
    return x, out


def _check_segment(x, out, pc, res_dtype, l, h):
    """Exact ranking and bf16-tolerance V_hat for one (layer, head)."""
    bias = lambda t, sl: None if t is None else _np(t[l:l + 1, h:h + 1])  # noqa: E731
    a = _np(x["a"][l // pc.group:l // pc.group + 1])
    d = pc.head_dim
    ref_vh = oracle.predicted_values(
        a, _np(x["b_l"][l:l + 1, h * d:(h + 1) * d]), _np(x["w_lin"][l:l + 1, h:h + 1]),
        _np(x["w1"][l:l + 1, h:h + 1]), _np(x["w2"][l:l + 1, h:h + 1]),
        bias(x["b1"], None), bias(x["b2"], None), group=1)[0, :, 0, :]
    vh = out["v_hat"][l, :, h, :].cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(vh - ref_vh, axis=1) / np.maximum(np.linalg.norm(ref_vh, axis=1), 1e-30)
    assert rel.max() <= TOL_BF16, rel.max()

    v = _np(x["v"][l:l + 1, :, h:h + 1, :])
    ref = oracle.prefill_rank(v, vh[None, :, None, :], pc.n_res, pc.block, res_dtype)
    np.testing.assert_array_equal(out["err"][l, h].cpu().numpy(), ref["err"][0, 0])
    np.testing.assert_array_equal(out["idx"][l, h].cpu().numpy(), ref["idx"][0, 0])
    np.testing.assert_array_equal(out["ptr"][l, h].cpu().numpy(), ref["ptr"][0, 0])
    if res_dtype in ("i8", "i2"):
        np.testing.assert_array_equal(out["val"][l, h].cpu().numpy(), ref["val"][0, 0])
        np.testing.assert_array_equal(out["scale"][l, h].cpu().numpy(), ref["scale"][0, 0])
    else:
        np.testing.assert_array_equal(_np(out["val"][l, h]), ref["val"][0, 0])
    return rel.max()


@pytest.mark.parametrize("res_dtype", ["bf16", "f32", "i8", "i2"])
def test_small_ragged_all_segments(res_dtype):
    pc = synth.PREFILL_CONFIGS["p_small_ragged"]          # T = 1000: a partial last block
    x, out = _launch(pc, res_dtype)
    worst = max(_check_segment(x, out, pc, res_dtype, l, h)
                for l in range(pc.n_slices) for h in range(pc.n_kv_heads))
    print(f"p_small_ragged {res_dtype}: max V_hat rel err {worst:.2e}", flush=True)


def test_mid_two_groups_all_segments():
    pc = synth.PREFILL_CONFIGS["p_mid"]                   # 8 layers: two key-factor groups
    x, out = _launch(pc, pc.res_dtype)
    worst = max(_check_segment(x, out, pc, pc.res_dtype, l, h)
                for l in range(pc.n_slices) for h in range(pc.n_kv_heads))
    print(f"p_mid: max V_hat rel err {worst:.2e}", flush=True)


@pytest.fixture(scope="module")
def p_c5_ranked():
    pc = synth.PREFILL_CONFIGS["p_c5"]                    # 32 x 131072 x 8 x 128
    x, out = _launch(pc, pc.res_dtype)
    yield pc, x, out
    del x, out
    torch.cuda.empty_cache()


def test_full_shape_sampled_v_hat(p_c5_ranked):
    """V_hat against the float64 predictor on sampled (layer, head) segments,
    with the exact ranking of those segments."""
    pc, x, out = p_c5_ranked
    for l, h in ((0, 0), (17, 5), (31, 7)):
        rel = _check_segment(x, out, pc, pc.res_dtype, l, h)
        print(f"p_c5 layer {l} head {h}: V_hat rel err {rel:.2e}", flush=True)


@pytest.mark.parametrize("part", range(4))
def test_full_shape_every_segment_ranked_exactly(p_c5_ranked, part):
    """Every (layer, head) segment at the full shape: errors, index set, block
    pointers and int8 residuals exactly the oracle's ranking of V against the
    V_hat the library returns, one layer (all heads) at a time; a quarter of
    the 32 layers per test."""
    pc, x, out = p_c5_ranked
    for l in range(8 * part, 8 * part + 8):
        v = _np(x["v"][l:l + 1])
        vh = out["v_hat"][l:l + 1].cpu().numpy().astype(np.float64)
        ref = oracle.prefill_rank(v, vh, pc.n_res, pc.block, pc.res_dtype)
        np.testing.assert_array_equal(out["err"][l].cpu().numpy(), ref["err"][0])
        np.testing.assert_array_equal(out["idx"][l].cpu().numpy(), ref["idx"][0])
        np.testing.assert_array_equal(out["ptr"][l].cpu().numpy(), ref["ptr"][0])
        np.testing.assert_array_equal(out["val"][l].cpu().numpy(), ref["val"][0])
        np.testing.assert_array_equal(out["scale"][l].cpu().numpy(), ref["scale"][0])
        print(f"layer {l}: 8 heads exact", flush=True)
