"""GPU parity of lowram_xkv_factorize against the float64 oracle's subspace
iteration run from the same starting block (same steps; the oracle's M is
exact, the library accumulates it in float32 per token chunk).

What is unique is the span of the basis, hence the reconstruction
K_l ~ A B_l; the basis itself is any orthonormal one of that span. So the
tests compare: the reconstruction from the library's bf16 A and B_l against
the oracle's (relative Frobenius error per layer within the bf16 tolerance),
the projector X X^T of the returned float64 basis against the oracle's, that
the basis is orthonormal, that B_l is the basis rounded to bf16, and that
A = C X on sampled rows. The error is also set against the Eckart-Young
optimum where the oracle's SVD of the keys is affordable.
"""
import numpy as np
import pytest
import torch

import long_context_decode_lowram_amd as L
import oracle
import synth

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_PROJ = 1e-4


def _run(xc):
    x = synth.gen_xkv_inputs(xc, "cuda")
    out = L.xkv_factorize(x["keys"], x["omega"], xc.n_iter, want_basis=True)
    torch.cuda.synchronize()
    return x, out


def _check(xc, x, out, *, projector=True, optimum=False):
    """x: keys [G, T, D] and omega of one problem; out: its outputs."""
    G, D, r = xc.n_layers, xc.width, xc.rank
    keys = [x["keys"][l].float().cpu().numpy().astype(np.float64) for l in range(G)]
    cat = np.concatenate(keys, axis=1)
    a_ref, bls_ref, x_ref = oracle.xkv_subspace_iteration(keys, r, x["omega"].cpu().numpy(), xc.n_iter)
    basis = out["basis"].cpu().numpy()
    live = np.linalg.norm(basis, axis=0) > 0
    gram = basis[:, live].T @ basis[:, live]
    assert np.abs(gram - np.eye(int(live.sum()))).max() < 1e-9
    np.testing.assert_array_equal(out["b_l"].float().cpu().numpy().reshape(G * D, r), oracle.round_bf16(basis))
    a = out["a"].float().cpu().numpy().astype(np.float64)
    b = out["b_l"].float().cpu().numpy().astype(np.float64)
    rows = np.unique(np.r_[0, xc.ctx_len - 1, np.random.default_rng(0).integers(0, xc.ctx_len, 64)])
    want = cat[rows] @ b.reshape(G * D, r)
    assert np.abs(a[rows] - want).max() <= 1e-2 * np.abs(want).max()
    worst = 0.0
    for l in range(G):
        rec = a @ b[l].T
        ref = oracle.reconstruct_keys(a_ref, bls_ref[l])
        rel = np.linalg.norm(rec - ref) / np.linalg.norm(ref)
        worst = max(worst, rel)
    assert worst <= TOL_BF16, worst
    proj = None
    if projector:
        proj = np.linalg.norm(basis @ basis.T - x_ref @ x_ref.T) / np.sqrt(r)
        assert proj <= TOL_PROJ, proj
    msg = f"{xc.name}: rebuild rel err {worst:.2e}" + ("" if proj is None else f", projector {proj:.2e}")
    if optimum:
        sv = np.linalg.svd(cat, compute_uv=False)
        tail = np.sqrt(np.sum(sv[r:] ** 2))
        err = np.linalg.norm(cat - cat @ basis @ basis.T)
        ref_err = np.linalg.norm(cat - cat @ x_ref @ x_ref.T)
        assert tail <= err <= 1.05 * tail and abs(err - ref_err) <= 1e-4 * ref_err
        msg += f", error / Eckart-Young optimum {err / tail:.4f}"
    print(msg, flush=True)


def test_small_ragged():
    xc = synth.XKV_CONFIGS["x_small_ragged"]              # T = 1000: a partial chunk and tile
    x, out = _run(xc)
    _check(xc, x, out, optimum=True)


def test_fewer_tokens_than_rank_is_exact():
    """T = 40 < r = 64: the basis holds the keys' whole row space, so the
    factors rebuild the keys to bf16 rounding."""
    xc = synth.XKV_CONFIGS["x_short"]
    x, out = _run(xc)
    _check(xc, x, out, projector=False)
    cat = torch.cat([x["keys"][l].float() for l in range(xc.n_layers)], dim=1).cpu().numpy()
    rec = np.concatenate([out["a"].float().cpu().numpy() @ out["b_l"][l].float().cpu().numpy().T
                          for l in range(xc.n_layers)], axis=1)
    assert np.linalg.norm(rec - cat) <= 1e-2 * np.linalg.norm(cat)


def test_zero_keys_give_zero_factors():
    xc = synth.XKV_CONFIGS["x_small_ragged"]
    keys = torch.zeros(xc.n_layers, 300, xc.width, dtype=torch.bfloat16, device="cuda")
    omega = torch.randn(xc.n, xc.rank, dtype=torch.float64, device="cuda")
    out = L.xkv_factorize(keys, omega, 2, want_basis=True)
    torch.cuda.synchronize()
    assert not out["a"].float().abs().sum().item() and not out["basis"].abs().sum().item()


def test_mid_four_layers():
    xc = synth.XKV_CONFIGS["x_mid"]                       # 4 x 1024 wide, T = 8192, r = 512
    x, out = _run(xc)
    _check(xc, x, out, optimum=True)


def test_max_rank():
    """r = 1024, the largest supported rank (sixteen 64-column Cholesky
    panels with a trailing update after each), on a ragged token count."""
    xc = synth.XKV_CONFIGS["x_rank_max"]
    x, out = _run(xc)
    _check(xc, x, out, optimum=True)


def test_full_shape():
    xc = synth.XKV_CONFIGS["x_llama_131k"]                # 4 Llama-3.1-8B layers, T = 131072, r = 512
    x, out = _run(xc)
    _check(xc, x, out)


def test_batch_of_groups():
    """Three independent groups in one call: each matches the oracle on its own."""
    xc = synth.XKV_CONFIGS["x_small_ragged"]
    x = synth.gen_xkv_inputs(xc, "cuda", batch=3)
    out = L.xkv_factorize(x["keys"], x["omega"], xc.n_iter, want_basis=True)
    torch.cuda.synchronize()
    assert out["a"].shape == (3, xc.ctx_len, xc.rank) and out["b_l"].shape == (3, xc.n_layers, xc.width, xc.rank)
    for b in range(3):
        _check(xc, {"keys": x["keys"][b], "omega": x["omega"]}, {k: v[b] for k, v in out.items()})


def test_bitwise_rerun():
    xc = synth.XKV_CONFIGS["x_small_ragged"]
    x, o1 = _run(xc)
    o2 = L.xkv_factorize(x["keys"], x["omega"], xc.n_iter, want_basis=True)
    torch.cuda.synchronize()
    assert torch.equal(o1["a"], o2["a"]) and torch.equal(o1["basis"], o2["basis"])
