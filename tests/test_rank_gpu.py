"""GPU parity of lowram_rank_residuals against the float64 oracle: errors
bit-exact, index sets and block pointers exact, stored residuals exact (the
rounding rules are fixed, so the encoded values must agree bit for bit)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _cases import np64

pytestmark = pytest.mark.gpu


def gpu_rank(v, vh, k, res_dtype):
    import long_context_decode_lowram_amd as L
    out = L.rank_residuals(v.cuda(), vh.cuda(), k, res_dtype, want_err=True)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.cpu()) for n, t in out.items()}


def compare(got, ref, res_dtype, segs=None):
    n_sl, n_kv = ref["idx"].shape[:2]
    for sl, h in (segs or [(s, hh) for s in range(n_sl) for hh in range(n_kv)]):
        gs, rs = (sl, h), (sl if segs is None else 0, h if segs is None else 0)
        assert np.array_equal(got["err"][gs].numpy().view(np.uint64), ref["err"][rs].view(np.uint64))
        np.testing.assert_array_equal(got["idx"][gs].numpy(), ref["idx"][rs])
        np.testing.assert_array_equal(got["ptr"][gs].numpy(), ref["ptr"][rs])
        if res_dtype in ("i8", "i2"):
            np.testing.assert_array_equal(got["val"][gs].numpy(), ref["val"][rs])
            np.testing.assert_array_equal(got["scale"][gs].numpy(), ref["scale"][rs])
        else:
            np.testing.assert_array_equal(np64(got["val"][gs]).astype(np.float64), ref["val"][rs])


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("res_dtype", ["f32", "bf16", "i8", "i2"])
def test_small_exact(in_dtype, res_dtype):
    rc = synth.RankConfig(3, 64 * 30 + 21, n_kv_heads=4, in_dtype=in_dtype, res_dtype=res_dtype)
    v, vh = synth.gen_rank_inputs(rc, "cpu")
    for k in (0, 1, rc.n_res, 777, rc.ctx_len):
        got = gpu_rank(v, vh, k, res_dtype)
        ref = oracle.rank_residuals(np64(v), np64(vh), k, 64, res_dtype)
        compare(got, ref, res_dtype)


def test_all_errors_equal_and_zero():
    v = torch.ones(1, 300, 2, 128, dtype=torch.bfloat16)
    vh = torch.zeros_like(v)
    got = gpu_rank(v, vh, 50, "i8")
    assert got["idx"][0, 0].tolist() == list(range(50))
    got = gpu_rank(vh, vh, 50, "bf16")              # every error zero: lowest indices, zero residuals
    assert got["idx"][0, 1].tolist() == list(range(50))
    assert not got["val"].float().abs().sum().item()


def test_two_bit_ties_and_zero_rows():
    """Residuals on the 2-bit rounding boundaries: with max|R| = 1.5 c and
    c = 2^-4 the scale is c exactly, so R = -c, 0, c give r/s + 1.5 = 0.5,
    1.5, 2.5, which round to the even codes 0, 2, 2; a zero row stores code 2
    and scale 0."""
    c = 2.0 ** -4
    row = np.resize(np.array([1.5, -1.5, -1.0, 0.0, 1.0, 0.5, -0.5, 0.25]) * c, 128)
    v = torch.zeros(1, 200, 2, 128, dtype=torch.float32)
    v[0, 7, 0] = torch.from_numpy(row)
    v[0, 9, 1] = torch.from_numpy(-row)
    vh = torch.zeros_like(v)
    got = gpu_rank(v, vh, 3, "i2")
    ref = oracle.rank_residuals(np64(v), np64(vh), 3, 64, "i2")
    compare(got, ref, "i2")
    q = oracle.unpack_i2(got["val"][0, 0, 1].numpy())
    assert got["idx"][0, 0].tolist() == [0, 1, 7] and got["scale"][0, 0, 2].item() == c
    assert oracle.unpack_i2(got["val"][0, 0, 2].numpy())[:8].tolist() == [3, 0, 0, 2, 2, 2, 1, 2]
    assert q.tolist() == [2] * 128 and got["scale"][0, 0, 1].item() == 0.0


@pytest.fixture(scope="module")
def c5_ranked():
    """32 slices x 131072 tokens x 8 heads, bf16 in, int8 residuals,
    k = 13107, ranked once on the GPU for the tests below."""
    rc = synth.RANK_C5
    torch.manual_seed(0)
    v, vh = synth.gen_rank_inputs(rc, "cuda")
    import long_context_decode_lowram_amd as L
    out = L.rank_residuals(v, vh, rc.n_res, "i8", want_err=True)
    torch.cuda.synchronize()
    yield rc, v, vh, out
    del v, vh, out
    torch.cuda.empty_cache()


def test_c5_full_shape_structure(c5_ranked):
    rc, v, vh, out = c5_ranked
    idx, ptr = out["idx"], out["ptr"]
    k = rc.n_res
    assert bool((idx[..., 1:] > idx[..., :-1]).all())
    assert bool((idx >= 0).all()) and bool((idx < rc.ctx_len).all())
    assert bool((ptr[..., -1] == k).all()) and bool((ptr[..., 0] == 0).all())
    assert torch.equal(ptr, synth.block_ptr_from_idx(idx, rc.ctx_len, 64))


@pytest.mark.parametrize("part", range(4))
def test_c5_full_shape_every_segment_exact(c5_ranked, part):
    """Index-exact at the full ranking shape: every (slice, head) segment's
    errors, index set, block pointers, int8 codes and scales against the
    oracle, one slice (all eight heads) at a time; a quarter of the 32 slices
    per test."""
    rc, v, vh, out = c5_ranked
    k = rc.n_res
    for sl in range(8 * part, 8 * part + 8):
        ref = oracle.rank_residuals(np64(v[sl:sl + 1]), np64(vh[sl:sl + 1]), k, 64, "i8")
        got = {n: (None if t is None else t[sl:sl + 1].cpu()) for n, t in out.items()}
        compare(got, ref, "i8")
        print(f"slice {sl}: 8 heads exact", flush=True)
