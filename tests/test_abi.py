"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, and rejects bad arguments with the
documented status before any HIP call."""
import ctypes
import os
import re

import pytest

import long_context_decode_lowram_amd as L
from long_context_decode_lowram_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lowram.h")
FAKE = 0x100000          # a 16-byte aligned non-NULL address; never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(lowram_[a-z_]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"lowram_decode_step", "lowram_decode_workspace_size", "lowram_rank_residuals",
            "lowram_rank_workspace_size", "lowram_status_string", "lowram_last_error"} <= set(names)
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_header_struct_layout_matches_binding():
    # Field order and count of the ctypes mirrors against the header text.
    text = open(HEADER).read()
    body = text[text.index("typedef struct lowram_decode_args"):text.index("} lowram_decode_args;")]
    fields = re.findall(r"\*?\s*([a-z_0-9]+)\s*[;,]", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert fields == [f[0] for f in B.DecodeArgs._fields_]
    body = text[text.index("typedef struct lowram_rank_args"):text.index("} lowram_rank_args;")]
    fields = re.findall(r"\*?\s*([a-z_0-9]+)\s*[;,]", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert fields == [f[0] for f in B.RankArgs._fields_]


def test_header_constants_match_binding():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+LOWRAM_([A-Z0-9_]+)\s+(-?\d+)", text))
    for name in ("F32", "BF16", "I8", "I2", "FLAG_GENERIC"):
        assert int(defs[name]) == getattr(B, name), name
    for name in ("OK", "ERR_ARG", "ERR_UNSUPPORTED", "ERR_WORKSPACE", "ERR_WINDOW_FULL", "ERR_EMPTY", "ERR_HIP"):
        assert int(defs[name]) == getattr(B, name), name


def test_status_strings():
    codes = [0, -1, -2, -3, -4, -5, -6]
    strs = [L.status_string(c) for c in codes]
    assert len(set(strs)) == len(codes)
    assert L.status_string(-99) == "unknown status"


def valid_decode():
    a = B.DecodeArgs()
    a.batch, a.ctx_len, a.n_q_heads, a.n_kv_heads, a.head_dim = 2, 1000, 32, 8, 128
    a.rank, a.mlp_hidden, a.block_size, a.n_res, a.n_sel, a.win_len, a.win_cap = 256, 64, 64, 200, 4, 3, 16
    a.act_dtype, a.a_dtype, a.res_dtype = B.BF16, B.BF16, B.BF16
    for n in ("q", "a", "b_l", "w_lin", "w1", "w2", "res_idx", "res_val", "res_blk_ptr", "sel",
              "win_k", "win_v", "out"):
        setattr(a, n, FAKE)
    return a


def call_decode(a):
    return L.lib().lowram_decode_step(ctypes.byref(a), None)


def test_decode_valid_args_stop_at_workspace():
    a = valid_decode()
    assert B.decode_workspace_size(a) > 0
    assert call_decode(a) == B.ERR_WORKSPACE
    a.workspace, a.workspace_bytes = FAKE, B.decode_workspace_size(a) - 1
    assert call_decode(a) == B.ERR_WORKSPACE
    assert "workspace" in L.last_error()


@pytest.mark.parametrize("field,value,status", [
    ("q", None, B.ERR_ARG),
    ("out", None, B.ERR_ARG),
    ("res_blk_ptr", None, B.ERR_ARG),
    ("win_k", None, B.ERR_ARG),
    ("q", FAKE + 4, B.ERR_ARG),                 # misaligned
    ("head_dim", 64, B.ERR_UNSUPPORTED),
    ("block_size", 32, B.ERR_UNSUPPORTED),
    ("rank", 250, B.ERR_UNSUPPORTED),
    ("mlp_hidden", 40, B.ERR_UNSUPPORTED),
    ("n_q_heads", 30, B.ERR_ARG),
    ("n_res", 1001, B.ERR_ARG),
    ("n_res", -1, B.ERR_ARG),
    ("n_sel", 17, B.ERR_ARG),                   # nb = 16
    ("win_len", 17, B.ERR_WINDOW_FULL),
    ("act_dtype", B.I8, B.ERR_ARG),
    ("a_dtype", 7, B.ERR_ARG),
    ("res_dtype", -1, B.ERR_ARG),
    ("batch", 0, B.ERR_ARG),
    ("a_dtype", B.I8, B.ERR_ARG),               # int8 A without a_scale
    ("res_dtype", B.I8, B.ERR_ARG),             # int8 residuals without res_scale
    ("res_dtype", B.I2, B.ERR_ARG),             # 2-bit residuals without res_scale
    ("res_dtype", 4, B.ERR_ARG),
    ("combine_stream", FAKE, B.ERR_ARG),        # a combine stream without its event
])
def test_decode_rejects(field, value, status):
    a = valid_decode()
    setattr(a, field, value)
    assert call_decode(a) == status
    assert L.last_error() != ""


def test_decode_empty_and_window_only():
    a = valid_decode()
    a.n_sel, a.win_len = 0, 0
    assert call_decode(a) == B.ERR_EMPTY
    a.win_len = 2                                # window only: valid, stops at workspace
    assert call_decode(a) == B.ERR_WORKSPACE
    a = valid_decode()
    a.ctx_len, a.n_res, a.win_len, a.sel = 0, 0, 0, None
    assert call_decode(a) == B.ERR_EMPTY


def test_decode_workspace_grows_with_batch_and_is_zero_when_invalid():
    a = valid_decode()
    n2 = B.decode_workspace_size(a)
    a.batch = 4
    assert B.decode_workspace_size(a) > n2
    a.head_dim = 64
    assert L.lib().lowram_decode_workspace_size(ctypes.byref(a)) == 0


def valid_rank():
    a = B.RankArgs()
    a.n_slices, a.ctx_len, a.n_kv_heads, a.head_dim, a.block_size, a.n_res = 2, 1000, 8, 128, 64, 100
    a.in_dtype, a.res_dtype = B.BF16, B.BF16
    for n in ("v", "v_hat", "res_idx", "res_val", "res_blk_ptr"):
        setattr(a, n, FAKE)
    return a


def call_rank(a):
    return L.lib().lowram_rank_residuals(ctypes.byref(a), None)


def test_rank_valid_args_stop_at_workspace():
    a = valid_rank()
    n = B.rank_workspace_size(a)
    assert n >= 2 * 8 * 1000 * 8            # errors kept in the workspace
    assert call_rank(a) == B.ERR_WORKSPACE
    a.err = FAKE
    assert B.rank_workspace_size(a) < n      # caller-provided err buffer


@pytest.mark.parametrize("field,value,status", [
    ("v", None, B.ERR_ARG), ("res_idx", None, B.ERR_ARG), ("res_val", None, B.ERR_ARG),
    ("head_dim", 96, B.ERR_UNSUPPORTED), ("block_size", 128, B.ERR_UNSUPPORTED),
    ("n_res", 1001, B.ERR_ARG), ("in_dtype", B.I8, B.ERR_ARG), ("res_dtype", B.I8, B.ERR_ARG),
    ("res_dtype", B.I2, B.ERR_ARG), ("res_dtype", 4, B.ERR_ARG), ("in_dtype", B.I2, B.ERR_ARG),
    ("n_slices", 0, B.ERR_ARG), ("v_hat", FAKE + 2, B.ERR_ARG),
])
def test_rank_rejects(field, value, status):
    a = valid_rank()
    setattr(a, field, value)
    assert call_rank(a) == status


def test_prefill_struct_layout_matches_binding():
    text = open(HEADER).read()
    body = text[text.index("typedef struct lowram_prefill_args"):text.index("} lowram_prefill_args;")]
    fields = re.findall(r"\*?\s*([a-z_0-9]+)\s*[;,]", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert fields == [f[0] for f in B.PrefillArgs._fields_]
    assert {"lowram_prefill_rank", "lowram_prefill_workspace_size", "lowram_xkv_factorize",
            "lowram_xkv_workspace_size"} <= set(declared_functions())


def valid_prefill():
    a = B.PrefillArgs()
    a.n_slices, a.group, a.ctx_len, a.n_kv_heads, a.head_dim = 4, 4, 1000, 2, 128
    a.rank, a.mlp_hidden, a.block_size, a.n_res = 256, 128, 64, 100
    a.act_dtype, a.res_dtype = B.BF16, B.BF16
    for n in ("a", "b_l", "w_lin", "w1", "w2", "v", "res_idx", "res_val", "res_blk_ptr"):
        setattr(a, n, FAKE)
    return a


def call_prefill(a):
    return L.lib().lowram_prefill_rank(ctypes.byref(a), None)


def test_prefill_valid_args_stop_at_workspace():
    a = valid_prefill()
    n = B.prefill_workspace_size(a)
    assert n >= 4 * 2 * 1000 * 8
    assert call_prefill(a) == B.ERR_WORKSPACE
    a.err = FAKE
    assert B.prefill_workspace_size(a) < n


@pytest.mark.parametrize("field,value,status", [
    ("a", None, B.ERR_ARG), ("w2", None, B.ERR_ARG), ("v", None, B.ERR_ARG), ("res_val", None, B.ERR_ARG),
    ("v_hat", FAKE + 8, B.ERR_ARG), ("b1", FAKE + 1, B.ERR_ARG),
    ("head_dim", 64, B.ERR_UNSUPPORTED), ("block_size", 32, B.ERR_UNSUPPORTED),
    ("rank", 96, B.ERR_UNSUPPORTED), ("mlp_hidden", 96, B.ERR_UNSUPPORTED), ("act_dtype", B.F32, B.ERR_UNSUPPORTED),
    ("ctx_len", 1 << 22, B.ERR_UNSUPPORTED),       # ctx_len * rank * 2 reaches 2^31
    ("n_res", 1001, B.ERR_ARG), ("res_dtype", B.I8, B.ERR_ARG), ("group", 0, B.ERR_ARG),
    ("res_dtype", B.I2, B.ERR_ARG), ("res_dtype", 4, B.ERR_ARG),
])
def test_prefill_rejects(field, value, status):
    a = valid_prefill()
    setattr(a, field, value)
    assert call_prefill(a) == status
    assert L.last_error() != ""


# ------------------------------------------------------- cross-layer factors
def valid_xkv():
    a = B.XkvArgs()
    a.n_batch, a.n_layers, a.ctx_len, a.width, a.rank, a.n_iter = 1, 4, 1000, 1024, 512, 3
    for n in ("keys", "omega", "a", "b_l"):
        setattr(a, n, FAKE)
    return a


def call_xkv(a):
    return L.lib().lowram_xkv_factorize(ctypes.byref(a), None)


def test_xkv_valid_args_stop_at_workspace():
    a = valid_xkv()
    n = B.xkv_workspace_size(a)
    assert n >= 4096 * 4096 * 8 + 2 * 4096 * 512 * 8      # M and the two basis blocks at least
    assert call_xkv(a) == B.ERR_WORKSPACE


def test_xkv_header_layout_matches_binding():
    text = open(HEADER).read()
    body = text[text.index("typedef struct lowram_xkv_args"):text.index("} lowram_xkv_args;")]
    fields = re.findall(r"\*?\s*([a-z_0-9]+)\s*[;,]", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert fields == [f[0] for f in B.XkvArgs._fields_]


@pytest.mark.parametrize("field,value,status", [
    ("keys", None, B.ERR_ARG), ("omega", None, B.ERR_ARG), ("a", None, B.ERR_ARG), ("b_l", None, B.ERR_ARG),
    ("basis", FAKE + 8, B.ERR_ARG), ("n_layers", 0, B.ERR_ARG), ("n_layers", 17, B.ERR_ARG), ("n_batch", 0, B.ERR_ARG),
    ("ctx_len", 0, B.ERR_ARG), ("width", 128, B.ERR_UNSUPPORTED), ("width", 1000, B.ERR_UNSUPPORTED),
    ("rank", 96, B.ERR_UNSUPPORTED), ("rank", 2048, B.ERR_UNSUPPORTED), ("n_iter", 0, B.ERR_ARG),
    ("n_iter", 17, B.ERR_ARG), ("ctx_len", 1 << 20, B.ERR_UNSUPPORTED),   # T * D * 2 reaches 2^31
])
def test_xkv_rejects(field, value, status):
    a = valid_xkv()
    setattr(a, field, value)
    assert call_xkv(a) == status
    assert L.last_error() != ""


def test_xkv_rank_above_width_rejected():
    a = valid_xkv()
    a.n_layers, a.width, a.rank = 1, 256, 320
    assert call_xkv(a) == B.ERR_UNSUPPORTED


# ------------------------------------------------- pseudoinverse and fit
def valid_pinv():
    a = B.PinvArgs()
    a.n_maps, a.hidden, a.head_dim = 4, 4096, 128
    for n in ("w_k", "w_v", "w_lin"):
        setattr(a, n, FAKE)
    return a


def valid_fit():
    a = B.FitArgs()
    a.n_layers, a.ctx_len, a.n_kv_heads, a.head_dim, a.mlp_hidden, a.n_steps, a.lr = 2, 1000, 8, 128, 256, 2, 0.05
    for n in ("keys", "v", "w_lin", "w1", "b1", "w2", "b2"):
        setattr(a, n, FAKE)
    return a


def test_pinv_and_fit_layouts_and_workspace():
    text = open(HEADER).read()
    for struct, cls in (("lowram_pinv_args", B.PinvArgs), ("lowram_fit_args", B.FitArgs)):
        body = text[text.index(f"typedef struct {struct}"):text.index(f"}} {struct};")]
        fields = re.findall(r"\*?\s*([a-z_0-9]+)\s*[;,]", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
        assert fields == [f[0] for f in cls._fields_]
    a = valid_pinv()
    assert L.lib().lowram_pinv_workspace_size(ctypes.byref(a)) >= 2 * 4 * 4096 * 128 * 8
    assert L.lib().lowram_pinv_value_map(ctypes.byref(a), None) == B.ERR_WORKSPACE
    f = valid_fit()
    assert L.lib().lowram_fit_workspace_size(ctypes.byref(f)) >= 2 * 16 * 1000 * 256 * 2
    assert L.lib().lowram_fit_predictor(ctypes.byref(f), None) == B.ERR_WORKSPACE


@pytest.mark.parametrize("field,value,status", [
    ("w_k", None, B.ERR_ARG), ("w_lin", None, B.ERR_ARG), ("n_maps", 0, B.ERR_ARG),
    ("head_dim", 64, B.ERR_UNSUPPORTED), ("hidden", 100, B.ERR_ARG), ("w_lin64", FAKE + 8, B.ERR_ARG),
])
def test_pinv_rejects(field, value, status):
    a = valid_pinv()
    setattr(a, field, value)
    assert L.lib().lowram_pinv_value_map(ctypes.byref(a), None) == status
    assert L.last_error() != ""


@pytest.mark.parametrize("field,value,status", [
    ("keys", None, B.ERR_ARG), ("b2", None, B.ERR_ARG), ("n_layers", 0, B.ERR_ARG), ("ctx_len", 0, B.ERR_ARG),
    ("head_dim", 64, B.ERR_UNSUPPORTED), ("mlp_hidden", 192, B.ERR_UNSUPPORTED), ("mlp_hidden", 2048, B.ERR_UNSUPPORTED),
    ("n_steps", -1, B.ERR_ARG), ("lr", float("nan"), B.ERR_ARG), ("lr", float("inf"), B.ERR_ARG),
    ("ctx_len", 1 << 21, B.ERR_UNSUPPORTED), ("losses", FAKE + 2, B.ERR_ARG),
])
def test_fit_rejects(field, value, status):
    a = valid_fit()
    setattr(a, field, value)
    assert L.lib().lowram_fit_predictor(ctypes.byref(a), None) == status
    assert L.last_error() != ""


# ------------------------------------------------- window, validate mode
def test_window_struct_layout_and_decode_tail_fields():
    text = open(HEADER).read()
    body = text[text.index("typedef struct lowram_window_args"):text.index("} lowram_window_args;")]
    fields = re.findall(r"\*?\s*([a-z_0-9]+)\s*[;,]", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert fields == [f[0] for f in B.WindowArgs._fields_]
    assert [f[0] for f in B.DecodeArgs._fields_][-2:] == ["win_len_dev", "check_flags"]
    defs = dict(re.findall(r"#define\s+LOWRAM_([A-Z0-9_]+)\s+(-?\d+)", text))
    for name in ("FLAG_VALIDATE", "CHECK_SEL_ORDER", "CHECK_RES_RANGE", "CHECK_RES_ORDER", "CHECK_RES_PTR",
                 "CHECK_WIN_LEN"):
        assert int(defs[name]) == getattr(B, name), name


@pytest.mark.parametrize("field,value,status", [
    ("flags", 4, B.ERR_ARG),                        # unknown flag bit
    ("flags", B.FLAG_VALIDATE, B.ERR_ARG),          # validate mode without check_flags
    ("win_len_dev", FAKE + 2, B.ERR_ARG),           # misaligned
    ("check_flags", FAKE + 1, B.ERR_ARG),
])
def test_decode_rejects_new_fields(field, value, status):
    a = valid_decode()
    setattr(a, field, value)
    assert call_decode(a) == status
    assert L.last_error() != ""


def test_decode_validate_and_device_window_stop_at_workspace():
    a = valid_decode()
    a.flags, a.check_flags, a.win_len_dev = B.FLAG_VALIDATE, FAKE, FAKE
    assert call_decode(a) == B.ERR_WORKSPACE


def valid_window():
    a = B.WindowArgs()
    a.n_layers, a.batch, a.width, a.win_cap, a.act_dtype = 32, 8, 1024, 1024, B.BF16
    for n in ("new_k", "new_v", "win_k", "win_v", "win_len_dev"):
        setattr(a, n, FAKE)
    return a


@pytest.mark.parametrize("field,value", [
    ("n_layers", 0), ("batch", 0), ("win_cap", 0), ("width", 4), ("width", 1020), ("act_dtype", B.I8),
    ("new_k", None), ("win_v", None), ("win_len_dev", None), ("win_k", FAKE + 8), ("win_len_dev", FAKE + 1),
])
def test_window_append_rejects(field, value):
    a = valid_window()
    setattr(a, field, value)
    assert L.lib().lowram_window_append(ctypes.byref(a), None) == B.ERR_ARG
    assert L.last_error() != ""


def test_prefill_rejects_v_beyond_32_bit_offsets():
    a = valid_prefill()
    a.rank, a.n_kv_heads, a.ctx_len = 64, 8, 1 << 20        # T*rank*2 = 2^27 fits, T*Hkv*d*2 = 2^31 does not
    assert call_prefill(a) == B.ERR_UNSUPPORTED
    assert "head_dim" in L.last_error()


# ------------------------------------------------- binding: tensor checks
def _decode_tensors(dtype=None):
    """A small, consistent set of host tensors for make_decode_args."""
    import torch
    act = dtype or torch.bfloat16
    B_, T, r, hkv, hq, d, h, k, n_sel, cap = 2, 200, 64, 2, 4, 128, 64, 7, 3, 8
    nb = -(-T // 64)
    t = dict(q=torch.zeros(B_, hq, d, dtype=act), a=torch.zeros(B_, T, r, dtype=act),
             b_l=torch.zeros(B_, hkv * d, r, dtype=act), w_lin=torch.zeros(B_, hkv, d, d, dtype=act),
             w1=torch.zeros(B_, hkv, h, d, dtype=act), w2=torch.zeros(B_, hkv, d, h, dtype=act),
             res_idx=torch.zeros(B_, hkv, k, dtype=torch.int32), res_val=torch.zeros(B_, hkv, k, d, dtype=act),
             res_blk_ptr=torch.zeros(B_, hkv, nb + 1, dtype=torch.int32), out=torch.zeros(B_, hq, d, dtype=act))
    kw = dict(b1=torch.zeros(B_, hkv, h, dtype=act), b2=torch.zeros(B_, hkv, d, dtype=act),
              sel=torch.zeros(B_, n_sel, dtype=torch.int32), keep=torch.ones(B_, nb, dtype=torch.uint8),
              win_k=torch.zeros(B_, cap, hkv * d, dtype=act), win_v=torch.zeros(B_, cap, hkv * d, dtype=act),
              win_len=3, stats=torch.zeros(B_, hkv, 2, dtype=torch.int32))
    return t, kw


def _make(t, kw):
    return L.make_decode_args(t["q"], t["a"], t["b_l"], t["w_lin"], t["w1"], t["w2"], t["res_idx"], t["res_val"],
                              t["res_blk_ptr"], t["out"], **kw)


def test_binding_accepts_consistent_shapes_then_rejects_host_tensors():
    t, kw = _decode_tensors()
    with pytest.raises(ValueError, match="device tensors only"):
        _make(t, kw)


def _mutations():
    import torch
    f32, bf, i8 = torch.float32, torch.bfloat16, torch.int8
    return [
        ("b_l", lambda t, kw: t.__setitem__("b_l", t["b_l"].to(f32)), "b_l: dtype"),          # fp32 weights, bf16 q
        ("q", lambda t, kw: t.__setitem__("q", t["q"].to(f32)), "dtype"),                     # fp32 q, bf16 weights
        ("w1", lambda t, kw: t.__setitem__("w1", t["w1"][:, :, :32].contiguous()), "w2: shape"),
        ("w2", lambda t, kw: t.__setitem__("w2", t["w2"][..., :32].contiguous()), "w2: shape"),
        ("w_lin", lambda t, kw: t.__setitem__("w_lin", t["w_lin"][:1].contiguous()), "w_lin: shape"),
        ("res_blk_ptr", lambda t, kw: t.__setitem__("res_blk_ptr", t["res_blk_ptr"][..., :-1].contiguous()),
         "res_blk_ptr: shape"),
        ("res_val", lambda t, kw: t.__setitem__("res_val", t["res_val"][:, :, :3].contiguous()), "res_val: shape"),
        ("res_idx", lambda t, kw: t.__setitem__("res_idx", t["res_idx"].to(torch.int64)), "res_idx: dtype"),
        ("out", lambda t, kw: t.__setitem__("out", t["out"][:, :2].contiguous()), "out: shape"),
        ("keep", lambda t, kw: kw.__setitem__("keep", kw["keep"][:, :-1].contiguous()), "keep: shape"),
        ("keep", lambda t, kw: kw.__setitem__("keep", kw["keep"].bool()), "keep: dtype"),
        ("sel", lambda t, kw: kw.__setitem__("sel", kw["sel"].to(torch.int64)), "sel"),
        ("win_v", lambda t, kw: kw.__setitem__("win_v", kw["win_v"][:, :4].contiguous()), "win_v: shape"),
        ("win_k", lambda t, kw: kw.__setitem__("win_k", None), "win_k"),
        ("b2", lambda t, kw: kw.__setitem__("b2", kw["b2"].to(f32)), "b2: dtype"),
        ("stats", lambda t, kw: kw.__setitem__("stats", kw["stats"][:, :1].contiguous()), "stats: shape"),
        ("a_scale", lambda t, kw: (t.__setitem__("a", t["a"].to(i8))), "a_scale is required"),
        ("a_scale", lambda t, kw: kw.__setitem__("a_scale", torch.ones(2, 200)), "int8 A only"),
        ("res_scale", lambda t, kw: t.__setitem__("res_val", t["res_val"].to(i8)), "res_scale is required"),
        ("res_scale", lambda t, kw: kw.__setitem__("res_scale", torch.ones(2, 2, 7)), "int8 and 2-bit"),
        ("win_len_dev", lambda t, kw: kw.__setitem__("win_len_dev", torch.zeros(2, dtype=torch.int32)),
         "win_len_dev: shape"),
    ]


@pytest.mark.parametrize("i", range(21))
def test_binding_rejects_inconsistent_tensors(i):
    name, mutate, msg = _mutations()[i]
    t, kw = _decode_tensors()
    mutate(t, kw)
    with pytest.raises(ValueError, match=msg):
        _make(t, kw)


def test_binding_rank_and_window_checks():
    import torch
    v = torch.zeros(2, 100, 2, 128, dtype=torch.bfloat16)
    idx = torch.zeros(2, 2, 10, dtype=torch.int32)
    val = torch.zeros(2, 2, 10, 128, dtype=torch.int8)
    scale = torch.zeros(2, 2, 10)
    ptr = torch.zeros(2, 2, 3, dtype=torch.int32)
    with pytest.raises(ValueError, match="v_hat: dtype"):
        L.make_rank_args(v, v.float(), 10, "i8", idx, val, scale, ptr)
    with pytest.raises(ValueError, match="res_val: dtype"):
        L.make_rank_args(v, v, 10, "bf16", idx, val, None, ptr)
    with pytest.raises(ValueError, match="res_blk_ptr: shape"):
        L.make_rank_args(v, v, 10, "i8", idx, val, scale, ptr[..., :2])
    with pytest.raises(ValueError, match="device tensors only"):
        L.make_rank_args(v, v, 10, "i8", idx, val, scale, ptr)
    wk = torch.zeros(3, 2, 16, 256, dtype=torch.bfloat16)
    nk = torch.zeros(3, 2, 256, dtype=torch.bfloat16)
    cnt = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="new_v: shape"):
        L.make_window_args(nk, nk[:2], wk, wk, cnt)
    with pytest.raises(ValueError, match="win_len_dev: shape"):
        L.make_window_args(nk, nk, wk, wk, cnt[:1])
    with pytest.raises(ValueError, match="device tensors only"):
        L.make_window_args(nk, nk, wk, wk, cnt)
