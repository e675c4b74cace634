"""GPU parity of the predictor's pseudoinverse start (lowram_pinv_value_map)
and test-time fit (lowram_fit_predictor) against the float64 oracle.

The pseudoinverse is computed in binary64 from the bf16 projections, so it
matches the oracle's to rounding level. The fit runs its products in bf16 with
float32 sums from float32 master weights, so after n steps the parameter
updates theta_n - theta_0 and the losses match the oracle's float64 gradient
descent from the same start within the bf16 tolerance (relative Frobenius
error of each parameter's update, relative error of each loss).
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
    return t.detach().float().cpu().numpy().astype(np.float64)


def test_pinv_matches_oracle():
    w_k, w_v = synth.gen_pinv_inputs(6, 1024, "cuda")
    w_lin, w64 = L.pinv_value_map(w_k, w_v, want_f64=True)
    torch.cuda.synchronize()
    for q in range(6):
        ref = oracle.pinv_value_map(_np(w_k[q]), _np(w_v[q]))
        got = w64[q].cpu().numpy()
        assert np.abs(got - ref).max() <= 1e-9 * np.abs(ref).max()
        np.testing.assert_array_equal(w_lin[q].float().cpu().numpy(), oracle.round_bf16(got))


def test_pinv_slim_case_recovers_values():
    """A square invertible W_K (hidden = d): k W_lin = x W_V exactly
    (explainer, Slim Attention paragraph), here to binary64 rounding."""
    g = torch.Generator(device="cuda").manual_seed(5)
    w_k = (torch.randn(2, 128, 128, generator=g, device="cuda") / 11.3).to(torch.bfloat16)
    w_v = (torch.randn(2, 128, 128, generator=g, device="cuda") / 11.3).to(torch.bfloat16)
    _, w64 = L.pinv_value_map(w_k, w_v, want_f64=True)
    torch.cuda.synchronize()
    x = np.random.default_rng(0).standard_normal((50, 128))
    for q in range(2):
        k = x @ _np(w_k[q])
        v = x @ _np(w_v[q])
        np.testing.assert_allclose(k @ w64[q].cpu().numpy().T, v, rtol=0, atol=1e-8 * np.abs(v).max())


def _fit(fc):
    x = synth.gen_fit_inputs(fc, "cuda")
    start = {n: x[n].clone() for n in ("w1", "b1", "w2", "b2")}
    losses = L.fit_predictor(x["keys"], x["v"], x["w_lin"], x["w1"], x["b1"], x["w2"], x["b2"], fc.n_steps, fc.lr)
    torch.cuda.synchronize()
    return x, start, losses


def _check(fc, x, start, losses, l, h):
    d = fc.head_dim
    k = _np(x["keys"][l, :, h * d:(h + 1) * d])
    v = _np(x["v"][l, :, h, :])
    w1, b1, w2, b2, ref_losses = oracle.fit_predictor(
        k, v, _np(x["w_lin"][l, h]), _np(start["w1"][l, h]), _np(start["b1"][l, h]), _np(start["w2"][l, h]),
        _np(start["b2"][l, h]), fc.lr, fc.n_steps)
    worst = 0.0
    for name, ref in (("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2)):
        d_ref = ref - _np(start[name][l, h])
        d_got = _np(x[name][l, h]) - _np(start[name][l, h])
        rel = np.linalg.norm(d_got - d_ref) / max(np.linalg.norm(d_ref), 1e-30)
        worst = max(worst, rel)
        assert rel <= TOL_BF16, (name, rel)
    got_l = losses[l, h].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got_l, ref_losses, rtol=TOL_BF16)
    assert got_l[-1] < got_l[0]
    return worst, got_l


def test_small_ragged_every_problem():
    fc = synth.FIT_CONFIGS["f_small_ragged"]        # T = 1000: partial token tiles and chunks
    x, start, losses = _fit(fc)
    worst = max(_check(fc, x, start, losses, l, h)[0] for l in range(fc.n_layers) for h in range(fc.n_kv_heads))
    print(f"f_small_ragged: worst update rel err {worst:.2e}", flush=True)


def test_wide_hidden_every_problem():
    fc = synth.FIT_CONFIGS["f_wide_ragged"]         # h = 384: the tiled forward, three hidden slices
    x, start, losses = _fit(fc)
    worst = max(_check(fc, x, start, losses, l, h)[0] for l in range(fc.n_layers) for h in range(fc.n_kv_heads))
    print(f"f_wide_ragged: worst update rel err {worst:.2e}", flush=True)


def test_mid_sampled():
    fc = synth.FIT_CONFIGS["f_mid"]
    x, start, losses = _fit(fc)
    for l, h in ((0, 0), (1, 7)):
        rel, ls = _check(fc, x, start, losses, l, h)
        print(f"f_mid ({l},{h}): update rel err {rel:.2e}, losses {ls}", flush=True)


def test_without_losses_same_parameters():
    """With no loss buffer the loss-only pass after the last step is skipped;
    the parameters are bit-identical to a run that reports the losses."""
    fc = synth.FIT_CONFIGS["f_small_ragged"]
    xa = synth.gen_fit_inputs(fc, "cuda")
    xb = {n: t.clone() for n, t in xa.items()}
    la = L.fit_predictor(xa["keys"], xa["v"], xa["w_lin"], xa["w1"], xa["b1"], xa["w2"], xa["b2"], fc.n_steps, fc.lr)
    lb = L.fit_predictor(xb["keys"], xb["v"], xb["w_lin"], xb["w1"], xb["b1"], xb["w2"], xb["b2"], fc.n_steps, fc.lr,
                         want_losses=False)
    torch.cuda.synchronize()
    assert lb is None and la.shape[-1] == fc.n_steps + 1
    for n in ("w1", "b1", "w2", "b2"):
        assert torch.equal(xa[n], xb[n]), n


def test_zero_steps_reports_the_start_loss():
    fc = synth.FIT_CONFIGS["f_small_ragged"]
    x = synth.gen_fit_inputs(fc, "cuda")
    w1 = x["w1"].clone()
    losses = L.fit_predictor(x["keys"], x["v"], x["w_lin"], x["w1"], x["b1"], x["w2"], x["b2"], 0, fc.lr)
    torch.cuda.synchronize()
    assert torch.equal(w1, x["w1"]) and losses.shape[-1] == 1
    d = fc.head_dim
    e = oracle.predict_values(_np(x["keys"][1, :, d:2 * d]), _np(x["w_lin"][1, 1]), _np(w1[1, 1]), _np(x["w2"][1, 1]),
                              _np(x["b1"][1, 1]), _np(x["b2"][1, 1])) - _np(x["v"][1, :, 1, :])
    ref = float(np.sum(e * e)) / fc.ctx_len
    assert abs(losses[1, 1, 0].item() - ref) <= TOL_BF16 * ref


def test_bitwise_rerun():
    fc = synth.FIT_CONFIGS["f_small_ragged"]
    x, _, l1 = _fit(fc)
    y, _, l2 = _fit(fc)
    assert torch.equal(l1, l2) and torch.equal(x["w1"], y["w1"]) and torch.equal(x["w2"], y["w2"])


def test_full_shape_sampled():
    """32 layers x 8 heads x 131072 tokens, h = 256, two steps: every
    problem's loss decreases, two sampled problems match the oracle."""
    fc = synth.FIT_CONFIGS["f_llama_131k"]
    x, start, losses = _fit(fc)
    assert bool((losses[:, :, -1] < losses[:, :, 0]).all())
    for l, h in ((0, 0), (31, 7)):
        rel, ls = _check(fc, x, start, losses, l, h)
        print(f"f_llama_131k ({l},{h}): update rel err {rel:.2e}, losses {ls}", flush=True)
