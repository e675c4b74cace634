"""ctypes binding over liblowram.so (argument marshalling only).

Every step of the decode and ranking paths runs in the library's HIP kernels;
torch provides device memory and the current stream. The library must be
built (``python -m long_context_decode_lowram_amd.build``); a missing library
is an error, there is no fallback.
"""
import ctypes
import os

import torch

# LOWRAM_LIBRARY names another build of the same library (the host-sanitizer
# build that the ABI tests run against); by default the in-tree one.
_LIB_PATH = os.environ.get("LOWRAM_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblowram.so")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_WINDOW_FULL, ERR_EMPTY, ERR_HIP = 0, -1, -2, -3, -4, -5, -6
F32, BF16, I8, I2 = 0, 1, 2, 3
FLAG_GENERIC, FLAG_VALIDATE = 1, 2
CHECK_SEL_ORDER, CHECK_RES_RANGE, CHECK_RES_ORDER, CHECK_RES_PTR, CHECK_WIN_LEN = 1, 2, 4, 8, 16
BLOCK = 64
NOALLOC_SCRATCH_BYTES = 64 << 20

# uint8 tensors carry 2-bit codes packed four per byte (residual rows [.., d/4]).
_DTYPE = {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.uint8: I2}
_RES_CODE = {"f32": F32, "bf16": BF16, "i8": I8, "i2": I2}
_RES_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "i2": torch.uint8}

_p = ctypes.c_void_p
_i = ctypes.c_int32


class DecodeArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in (
        "batch", "ctx_len", "n_q_heads", "n_kv_heads", "head_dim", "rank", "mlp_hidden", "block_size",
        "n_res", "n_sel", "win_len", "win_cap", "act_dtype", "a_dtype", "res_dtype", "flags")] + [
        (n, _p) for n in (
        "q", "a", "a_scale", "b_l", "w_lin", "w1", "b1", "w2", "b2", "res_idx", "res_val", "res_scale",
        "res_blk_ptr", "sel", "keep", "win_k", "win_v", "out", "stats", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t), ("ev_main_begin", _p), ("ev_main_end", _p),
        ("combine_stream", _p), ("combine_ready", _p), ("win_len_dev", _p), ("check_flags", _p)]


class WindowArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("n_layers", "batch", "width", "win_cap", "act_dtype")] + [
        (n, _p) for n in ("new_k", "new_v", "win_k", "win_v", "win_len_dev")]


class RankArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in (
        "n_slices", "ctx_len", "n_kv_heads", "head_dim", "block_size", "n_res", "in_dtype", "res_dtype")] + [
        (n, _p) for n in ("v", "v_hat", "res_idx", "res_val", "res_scale", "res_blk_ptr", "err", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t), ("ev_main_begin", _p), ("ev_main_end", _p)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in (
        "n_slices", "group", "ctx_len", "n_kv_heads", "head_dim", "rank", "mlp_hidden", "block_size",
        "n_res", "act_dtype", "res_dtype")] + [
        (n, _p) for n in ("a", "b_l", "w_lin", "w1", "b1", "w2", "b2", "v", "res_idx", "res_val",
                          "res_scale", "res_blk_ptr", "err", "v_hat", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t), ("ev_main_begin", _p), ("ev_main_end", _p)]


class XkvArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("n_batch", "n_layers", "ctx_len", "width", "rank", "n_iter")] + [
        (n, _p) for n in ("keys", "omega", "a", "b_l", "basis", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t), ("ev_main_begin", _p), ("ev_main_end", _p)]


class PinvArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("n_maps", "hidden", "head_dim")] + [
        (n, _p) for n in ("w_k", "w_v", "w_lin", "w_lin64", "workspace")] + [("workspace_bytes", ctypes.c_size_t)]


class FitArgs(ctypes.Structure):
    _fields_ = [(n, _i) for n in ("n_layers", "ctx_len", "n_kv_heads", "head_dim", "mlp_hidden", "n_steps")] + [
        ("lr", ctypes.c_float)] + [
        (n, _p) for n in ("keys", "v", "w_lin", "w1", "b1", "w2", "b2", "losses", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t), ("ev_main_begin", _p), ("ev_main_end", _p)]


class LowramError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"liblowram status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m long_context_decode_lowram_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        L.lowram_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _p]
        L.lowram_decode_step.restype = ctypes.c_int
        L.lowram_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeArgs)]
        L.lowram_decode_workspace_size.restype = ctypes.c_size_t
        L.lowram_decode_step_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), _p]
        L.lowram_decode_step_noalloc.restype = ctypes.c_int
        L.lowram_window_append.argtypes = [ctypes.POINTER(WindowArgs), _p]
        L.lowram_window_append.restype = ctypes.c_int
        L.lowram_rank_residuals.argtypes = [ctypes.POINTER(RankArgs), _p]
        L.lowram_rank_residuals.restype = ctypes.c_int
        L.lowram_rank_workspace_size.argtypes = [ctypes.POINTER(RankArgs)]
        L.lowram_rank_workspace_size.restype = ctypes.c_size_t
        L.lowram_prefill_rank.argtypes = [ctypes.POINTER(PrefillArgs), _p]
        L.lowram_prefill_rank.restype = ctypes.c_int
        L.lowram_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs)]
        L.lowram_prefill_workspace_size.restype = ctypes.c_size_t
        L.lowram_xkv_factorize.argtypes = [ctypes.POINTER(XkvArgs), _p]
        L.lowram_xkv_factorize.restype = ctypes.c_int
        L.lowram_xkv_workspace_size.argtypes = [ctypes.POINTER(XkvArgs)]
        L.lowram_xkv_workspace_size.restype = ctypes.c_size_t
        for name, st in (("pinv_value_map", PinvArgs), ("fit_predictor", FitArgs)):
            getattr(L, "lowram_" + name).argtypes = [ctypes.POINTER(st), _p]
            getattr(L, "lowram_" + name).restype = ctypes.c_int
        for name, st in (("pinv", PinvArgs), ("fit", FitArgs)):
            getattr(L, f"lowram_{name}_workspace_size").argtypes = [ctypes.POINTER(st)]
            getattr(L, f"lowram_{name}_workspace_size").restype = ctypes.c_size_t
        L.lowram_status_string.argtypes = [ctypes.c_int]
        L.lowram_status_string.restype = ctypes.c_char_p
        L.lowram_last_error.argtypes = []
        L.lowram_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status):
    return lib().lowram_status_string(status).decode()


def last_error():
    return lib().lowram_last_error().decode()


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to liblowram must be contiguous")
    return t.data_ptr()


def _dt(t, name):
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}") from None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _want(name, t, shape, dtypes):
    """Raise ValueError unless tensor ``t`` has exactly ``shape`` and one of ``dtypes``."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {[str(x) for x in dtypes]}")


def _same_gpu(named):
    """Every tensor on the CUDA (HIP) device of the first one: the library
    reads device pointers only, so a host tensor must never reach it."""
    first = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}; liblowram takes device tensors only")
        if first is None:
            first = t.device
        elif t.device != first:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {first}")


_ACT = (torch.float32, torch.bfloat16)
_I32 = (torch.int32,)


def _check_decode(q, a, b_l, w_lin, w1, w2, res_idx, res_val, res_blk_ptr, out, a_scale, b1, b2, res_scale,
                  sel, keep, win_k, win_v, win_len, stats, win_len_dev, check_flags, workspace):
    """Shapes, dtypes and device of every decode tensor against the shapes the
    header documents, derived from (B, Hq, d) of q, (T, r) of a, Hkv from b_l,
    h from w1, k from res_idx; raises ValueError before anything is launched."""
    if q.dim() != 3 or a.dim() != 3 or b_l.dim() != 3 or w1.dim() != 4 or res_idx.dim() != 3:
        raise ValueError("q, a, b_l must be 3-D, w1 4-D and res_idx 3-D")
    B, Hq, d = q.shape
    T, r = a.shape[1], a.shape[2]
    if b_l.shape[1] % d:
        raise ValueError(f"b_l: {b_l.shape[1]} rows is not a multiple of head_dim {d}")
    hkv, h, k = b_l.shape[1] // d, w1.shape[2], res_idx.shape[2]
    nb = -(-T // BLOCK)
    act = q.dtype
    if act not in _ACT:
        raise ValueError(f"q: dtype {act}, expected float32 or bfloat16")
    _want("a", a, (B, T, r), (torch.float32, torch.bfloat16, torch.int8))
    if a.dtype == torch.int8:
        _want("a_scale", a_scale, (B, T), (torch.float32,))
    elif a_scale is not None:
        raise ValueError("a_scale is for int8 A only")
    _want("b_l", b_l, (B, hkv * d, r), (act,))
    _want("w_lin", w_lin, (B, hkv, d, d), (act,))
    _want("w1", w1, (B, hkv, h, d), (act,))
    _want("w2", w2, (B, hkv, d, h), (act,))
    if b1 is not None:
        _want("b1", b1, (B, hkv, h), (act,))
    if b2 is not None:
        _want("b2", b2, (B, hkv, d), (act,))
    _want("res_idx", res_idx, (B, hkv, k), _I32)
    if res_val is None or res_val.dtype not in _DTYPE:
        raise ValueError("res_val must be float32, bfloat16, int8 or uint8 (2-bit codes)")
    _want("res_val", res_val, (B, hkv, k, d // 4 if res_val.dtype == torch.uint8 else d), (res_val.dtype,))
    if res_val.dtype in (torch.int8, torch.uint8):
        if k > 0 or res_scale is not None:
            _want("res_scale", res_scale, (B, hkv, k), (torch.float32,))
    elif res_scale is not None:
        raise ValueError("res_scale is for int8 and 2-bit residuals only")
    _want("res_blk_ptr", res_blk_ptr, (B, hkv, nb + 1), _I32)
    if sel is not None:
        if sel.dim() != 2 or sel.shape[0] != B or sel.dtype != torch.int32:
            raise ValueError(f"sel: expected int32 [B={B}, n_sel], got {sel.dtype} {tuple(sel.shape)}")
    if keep is not None:
        _want("keep", keep, (B, nb), (torch.uint8,))
    if win_k is not None or win_v is not None:
        if win_k is None or win_k.dim() != 3:
            raise ValueError("win_k: expected [B, win_cap, Hkv*d]")
        _want("win_k", win_k, (B, win_k.shape[1], hkv * d), (act,))
        _want("win_v", win_v, tuple(win_k.shape), (act,))
    elif win_len:
        raise ValueError("win_len > 0 needs win_k and win_v")
    _want("out", out, (B, Hq, d), (act,))
    if stats is not None:
        _want("stats", stats, (B, hkv, 2), _I32)
    if win_len_dev is not None:
        _want("win_len_dev", win_len_dev, (1,), _I32)
    if check_flags is not None:
        _want("check_flags", check_flags, (1,), (torch.int32, torch.uint32) if hasattr(torch, "uint32") else _I32)
    if workspace is not None and workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    _same_gpu((("q", q), ("a", a), ("a_scale", a_scale), ("b_l", b_l), ("w_lin", w_lin), ("w1", w1),
               ("w2", w2), ("b1", b1), ("b2", b2), ("res_idx", res_idx), ("res_val", res_val),
               ("res_scale", res_scale), ("res_blk_ptr", res_blk_ptr), ("sel", sel), ("keep", keep),
               ("win_k", win_k), ("win_v", win_v), ("out", out), ("stats", stats),
               ("win_len_dev", win_len_dev), ("check_flags", check_flags), ("workspace", workspace)))


def make_decode_args(q, a, b_l, w_lin, w1, w2, res_idx, res_val, res_blk_ptr, out, *, a_scale=None,
                     b1=None, b2=None, res_scale=None, sel=None, keep=None, win_k=None, win_v=None,
                     win_len=0, stats=None, workspace=None, generic=False, events=None, win_len_dev=None,
                     validate=None):
    """Fill a DecodeArgs from tensors (shapes as documented in lowram.h).
    ``workspace`` may be None to size it first with ``decode_workspace_size``.
    ``win_len_dev`` (int32 [1] on the device) makes the kernels read the window
    length at run time, ``win_len`` then being its upper bound; ``validate``
    (int32 [1] on the device, cleared by the caller) turns on the validate
    mode, whose defect bits (CHECK_*) land there. Every tensor's shape, dtype
    and device is checked first (ValueError)."""
    _check_decode(q, a, b_l, w_lin, w1, w2, res_idx, res_val, res_blk_ptr, out, a_scale, b1, b2, res_scale,
                  sel, keep, win_k, win_v, win_len, stats, win_len_dev, validate, workspace)
    B, Hq, d = q.shape
    T, r = a.shape[1], a.shape[2]
    args = DecodeArgs()
    args.batch, args.ctx_len, args.n_q_heads = B, T, Hq
    args.n_kv_heads = b_l.shape[1] // d
    args.head_dim, args.rank, args.mlp_hidden, args.block_size = d, r, w1.shape[2], BLOCK
    args.n_res = res_idx.shape[-1]
    args.n_sel = 0 if sel is None else sel.shape[1]
    args.win_len = win_len
    args.win_cap = 0 if win_k is None else win_k.shape[1]
    args.act_dtype = _dt(q, "q")
    args.a_dtype = _dt(a, "a")
    args.res_dtype = _dt(res_val, "res_val")
    args.flags = (FLAG_GENERIC if generic else 0) | (FLAG_VALIDATE if validate is not None else 0)
    for name, t in (("q", q), ("a", a), ("a_scale", a_scale), ("b_l", b_l), ("w_lin", w_lin), ("w1", w1),
                    ("b1", b1), ("w2", w2), ("b2", b2), ("res_idx", res_idx), ("res_val", res_val),
                    ("res_scale", res_scale), ("res_blk_ptr", res_blk_ptr), ("sel", sel), ("keep", keep),
                    ("win_k", win_k), ("win_v", win_v), ("out", out), ("stats", stats), ("workspace", workspace),
                    ("win_len_dev", win_len_dev), ("check_flags", validate)):
        setattr(args, name, _ptr(t))
    args.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if events is not None:
        args.ev_main_begin, args.ev_main_end = events
    return args


def decode_workspace_size(args):
    n = lib().lowram_decode_workspace_size(ctypes.byref(args))
    if n == 0:
        raise LowramError(ERR_ARG, last_error() or "invalid arguments")
    return n


def decode_launch(args, stream=None):
    rc = lib().lowram_decode_step(ctypes.byref(args), _stream(stream))
    if rc != OK:
        raise LowramError(rc, last_error())


def decode_launch_noalloc(args, stream=None):
    """lowram_decode_step_noalloc: the step with the library's static scratch
    array in place of a workspace (args.workspace is ignored)."""
    rc = lib().lowram_decode_step_noalloc(ctypes.byref(args), _stream(stream))
    if rc != OK:
        raise LowramError(rc, last_error())


def decode_step(q, a, b_l, w_lin, w1, w2, res_idx, res_val, res_blk_ptr, *, out=None, workspace=None,
                stream=None, **kw):
    """One layer's decode step; returns ``out`` [B, Hq, d]. A workspace is
    allocated with torch when none is given."""
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    args = make_decode_args(q, a, b_l, w_lin, w1, w2, res_idx, res_val, res_blk_ptr, out, **kw)
    if workspace is None:
        workspace = torch.empty(decode_workspace_size(args), dtype=torch.uint8, device=q.device)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel()
    decode_launch(args, stream)
    return out


def make_window_args(new_k, new_v, win_k, win_v, win_len_dev):
    """Arguments of lowram_window_append: new_k, new_v [L, B, width];
    win_k, win_v [L, B, win_cap, width] (layer l's buffers are what its decode
    call takes); win_len_dev int32 [L] fill counts on the device."""
    if win_k.dim() != 4:
        raise ValueError("win_k: expected [n_layers, B, win_cap, width]")
    Lw, B, cap, width = win_k.shape
    if win_k.dtype not in _ACT:
        raise ValueError(f"win_k: dtype {win_k.dtype}, expected float32 or bfloat16")
    _want("win_v", win_v, (Lw, B, cap, width), (win_k.dtype,))
    _want("new_k", new_k, (Lw, B, width), (win_k.dtype,))
    _want("new_v", new_v, (Lw, B, width), (win_k.dtype,))
    _want("win_len_dev", win_len_dev, (Lw,), _I32)
    _same_gpu((("win_k", win_k), ("win_v", win_v), ("new_k", new_k), ("new_v", new_v),
               ("win_len_dev", win_len_dev)))
    args = WindowArgs()
    args.n_layers, args.batch, args.width, args.win_cap = Lw, B, width, cap
    args.act_dtype = _DTYPE[win_k.dtype]
    for name, t in (("new_k", new_k), ("new_v", new_v), ("win_k", win_k), ("win_v", win_v),
                    ("win_len_dev", win_len_dev)):
        setattr(args, name, _ptr(t))
    return args


def window_launch(args, stream=None):
    rc = lib().lowram_window_append(ctypes.byref(args), _stream(stream))
    if rc != OK:
        raise LowramError(rc, last_error())


def window_append(new_k, new_v, win_k, win_v, win_len_dev, *, stream=None):
    """Append one exact key/value row per (layer, sequence) at each layer's
    fill count and advance the counts (lowram_window_append)."""
    window_launch(make_window_args(new_k, new_v, win_k, win_v, win_len_dev), stream)


def make_rank_args(v, v_hat, n_res, res_dtype, res_idx, res_val, res_scale, res_blk_ptr, *, err=None,
                   workspace=None, events=None):
    """Arguments of lowram_rank_residuals; shapes, dtypes and devices are
    checked against v [Lr, T, Hkv, d] first (ValueError)."""
    if v.dim() != 4:
        raise ValueError("v: expected [Lr, T, Hkv, d]")
    Lr, T, Hkv, d = v.shape
    if v.dtype not in _ACT:
        raise ValueError(f"v: dtype {v.dtype}, expected float32 or bfloat16")
    if res_dtype not in _RES_CODE:
        raise ValueError(f"res_dtype must be one of {sorted(_RES_CODE)}")
    nb = -(-T // BLOCK)
    _want("v_hat", v_hat, tuple(v.shape), (v.dtype,))
    if n_res > 0 or res_idx is not None:
        _want("res_idx", res_idx, (Lr, Hkv, n_res), _I32)
        _want("res_val", res_val, (Lr, Hkv, n_res, d // 4 if res_dtype == "i2" else d), (_RES_TORCH[res_dtype],))
    if res_dtype in ("i8", "i2") and (n_res > 0 or res_scale is not None):
        _want("res_scale", res_scale, (Lr, Hkv, n_res), (torch.float32,))
    _want("res_blk_ptr", res_blk_ptr, (Lr, Hkv, nb + 1), _I32)
    if err is not None:
        _want("err", err, (Lr, Hkv, T), (torch.float64,))
    _same_gpu((("v", v), ("v_hat", v_hat), ("res_idx", res_idx), ("res_val", res_val), ("res_scale", res_scale),
               ("res_blk_ptr", res_blk_ptr), ("err", err), ("workspace", workspace)))
    args = RankArgs()
    args.n_slices, args.ctx_len, args.n_kv_heads, args.head_dim = Lr, T, Hkv, d
    args.block_size, args.n_res = BLOCK, n_res
    args.in_dtype = _dt(v, "v")
    args.res_dtype = _RES_CODE[res_dtype]
    for name, t in (("v", v), ("v_hat", v_hat), ("res_idx", res_idx), ("res_val", res_val),
                    ("res_scale", res_scale), ("res_blk_ptr", res_blk_ptr), ("err", err),
                    ("workspace", workspace)):
        setattr(args, name, _ptr(t))
    args.workspace_bytes = 0 if workspace is None else workspace.numel()
    if events is not None:
        args.ev_main_begin, args.ev_main_end = events
    return args


def rank_workspace_size(args):
    n = lib().lowram_rank_workspace_size(ctypes.byref(args))
    if n == 0:
        raise LowramError(ERR_ARG, last_error() or "invalid arguments")
    return n


def rank_launch(args, stream=None):
    rc = lib().lowram_rank_residuals(ctypes.byref(args), _stream(stream))
    if rc != OK:
        raise LowramError(rc, last_error())


def _res_store(Lr, Hkv, n_res, d, res_dtype, dev):
    """Residual value rows (i2: d/4 packed bytes) and per-row scales (i8, i2)."""
    width = d // 4 if res_dtype == "i2" else d
    val = torch.empty(Lr, Hkv, n_res, width, dtype=_RES_TORCH[res_dtype], device=dev)
    scale = torch.empty(Lr, Hkv, n_res, dtype=torch.float32, device=dev) if res_dtype in ("i8", "i2") else None
    return val, scale


def rank_residuals(v, v_hat, n_res, res_dtype, *, want_err=False, workspace=None, stream=None):
    """Residual store for V, V_hat [Lr, T, Hkv, d]. Returns a dict with idx,
    val, scale (int8 and 2-bit only), ptr and err (when ``want_err``)."""
    Lr, T, Hkv, d = v.shape
    dev = v.device
    nb = -(-T // BLOCK)
    out = {
        "idx": torch.empty(Lr, Hkv, n_res, dtype=torch.int32, device=dev),
        **dict(zip(("val", "scale"), _res_store(Lr, Hkv, n_res, d, res_dtype, dev))),
        "ptr": torch.empty(Lr, Hkv, nb + 1, dtype=torch.int32, device=dev),
        "err": torch.empty(Lr, Hkv, T, dtype=torch.float64, device=dev) if want_err else None,
    }
    args = make_rank_args(v, v_hat, n_res, res_dtype, out["idx"], out["val"], out["scale"], out["ptr"],
                          err=out["err"])
    if workspace is None:
        workspace = torch.empty(rank_workspace_size(args), dtype=torch.uint8, device=dev)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel()
    rank_launch(args, stream)
    return out


def make_prefill_args(a, b_l, w_lin, w1, w2, v, n_res, res_dtype, res_idx, res_val, res_scale, res_blk_ptr, *,
                      group=4, b1=None, b2=None, err=None, v_hat=None, workspace=None, events=None):
    """Arguments of lowram_prefill_rank. a [ceil(Lr/group), T, r], b_l [Lr, Hkv*d, r],
    w_lin [Lr, Hkv, d, d], w1 [Lr, Hkv, h, d], w2 [Lr, Hkv, d, h], v [Lr, T, Hkv, d],
    all bf16; shapes, dtypes and devices are checked first (ValueError)."""
    if v.dim() != 4 or a.dim() != 3 or w1.dim() != 4:
        raise ValueError("v must be 4-D, a 3-D and w1 4-D")
    Lr, T, Hkv, d = v.shape
    if res_dtype not in _RES_CODE:
        raise ValueError(f"res_dtype must be one of {sorted(_RES_CODE)}")
    bf, r, h, nb = (torch.bfloat16,), a.shape[-1], w1.shape[-2], -(-T // BLOCK)
    _want("v", v, (Lr, T, Hkv, d), bf)
    _want("a", a, (-(-Lr // group) if group > 0 else a.shape[0], T, r), bf)
    _want("b_l", b_l, (Lr, Hkv * d, r), bf)
    _want("w_lin", w_lin, (Lr, Hkv, d, d), bf)
    _want("w1", w1, (Lr, Hkv, h, d), bf)
    _want("w2", w2, (Lr, Hkv, d, h), bf)
    if b1 is not None:
        _want("b1", b1, (Lr, Hkv, h), bf)
    if b2 is not None:
        _want("b2", b2, (Lr, Hkv, d), bf)
    if n_res > 0 or res_idx is not None:
        _want("res_idx", res_idx, (Lr, Hkv, n_res), _I32)
        _want("res_val", res_val, (Lr, Hkv, n_res, d // 4 if res_dtype == "i2" else d), (_RES_TORCH[res_dtype],))
    if res_dtype in ("i8", "i2") and (n_res > 0 or res_scale is not None):
        _want("res_scale", res_scale, (Lr, Hkv, n_res), (torch.float32,))
    _want("res_blk_ptr", res_blk_ptr, (Lr, Hkv, nb + 1), _I32)
    if err is not None:
        _want("err", err, (Lr, Hkv, T), (torch.float64,))
    if v_hat is not None:
        _want("v_hat", v_hat, (Lr, T, Hkv, d), (torch.float32,))
    _same_gpu((("v", v), ("a", a), ("b_l", b_l), ("w_lin", w_lin), ("w1", w1), ("w2", w2), ("b1", b1), ("b2", b2),
               ("res_idx", res_idx), ("res_val", res_val), ("res_scale", res_scale), ("res_blk_ptr", res_blk_ptr),
               ("err", err), ("v_hat", v_hat), ("workspace", workspace)))
    args = PrefillArgs()
    args.n_slices, args.group, args.ctx_len, args.n_kv_heads, args.head_dim = Lr, group, T, Hkv, d
    args.rank, args.mlp_hidden, args.block_size, args.n_res = a.shape[-1], w1.shape[-2], BLOCK, n_res
    args.act_dtype = _dt(v, "v")
    args.res_dtype = _RES_CODE[res_dtype]
    for name, t in (("a", a), ("b_l", b_l), ("w_lin", w_lin), ("w1", w1), ("b1", b1), ("w2", w2),
                    ("b2", b2), ("v", v), ("res_idx", res_idx), ("res_val", res_val),
                    ("res_scale", res_scale), ("res_blk_ptr", res_blk_ptr), ("err", err),
                    ("v_hat", v_hat), ("workspace", workspace)):
        setattr(args, name, _ptr(t))
    args.workspace_bytes = 0 if workspace is None else workspace.numel()
    if events is not None:
        args.ev_main_begin, args.ev_main_end = events
    return args


def prefill_workspace_size(args):
    n = lib().lowram_prefill_workspace_size(ctypes.byref(args))
    if n == 0:
        raise LowramError(ERR_ARG, last_error() or "invalid arguments")
    return n


def prefill_launch(args, stream=None):
    rc = lib().lowram_prefill_rank(ctypes.byref(args), _stream(stream))
    if rc != OK:
        raise LowramError(rc, last_error())


def prefill_rank(a, b_l, w_lin, w1, w2, v, n_res, res_dtype, *, group=4, b1=None, b2=None, want_err=False,
                 want_v_hat=False, workspace=None, stream=None):
    """Fused prefill ranking: the residual store of V against the values the
    cache's own predictor gives (computed in the library). Returns a dict like
    ``rank_residuals`` plus ``v_hat`` (fp32, when ``want_v_hat``)."""
    Lr, T, Hkv, d = v.shape
    dev = v.device
    nb = -(-T // BLOCK)
    out = {
        "idx": torch.empty(Lr, Hkv, n_res, dtype=torch.int32, device=dev),
        **dict(zip(("val", "scale"), _res_store(Lr, Hkv, n_res, d, res_dtype, dev))),
        "ptr": torch.empty(Lr, Hkv, nb + 1, dtype=torch.int32, device=dev),
        "err": torch.empty(Lr, Hkv, T, dtype=torch.float64, device=dev) if want_err else None,
        "v_hat": torch.empty(Lr, T, Hkv, d, dtype=torch.float32, device=dev) if want_v_hat else None,
    }
    args = make_prefill_args(a, b_l, w_lin, w1, w2, v, n_res, res_dtype, out["idx"], out["val"], out["scale"],
                             out["ptr"], group=group, b1=b1, b2=b2, err=out["err"], v_hat=out["v_hat"])
    if workspace is None:
        workspace = torch.empty(prefill_workspace_size(args), dtype=torch.uint8, device=dev)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel()
    prefill_launch(args, stream)
    return out


def make_xkv_args(keys, omega, n_iter, a, b_l, *, basis=None, workspace=None, events=None):
    """Fill an XkvArgs: keys [Bt, G, T, D] (or one problem [G, T, D]) bf16,
    omega [G*D, r] float64, a [Bt, T, r] and b_l [Bt, G, D, r] bf16 outputs,
    basis [Bt, G*D, r] float64 or None."""
    if keys.dim() == 3:
        keys = keys.unsqueeze(0)
    Bt, G, T, D = keys.shape
    if keys.dtype != torch.bfloat16 or omega.dtype != torch.float64:
        raise ValueError("keys must be bfloat16 and omega float64")
    args = XkvArgs()
    args.n_batch, args.n_layers, args.ctx_len, args.width = Bt, G, T, D
    args.rank, args.n_iter = omega.shape[1], n_iter
    for name, t in (("keys", keys), ("omega", omega), ("a", a), ("b_l", b_l), ("basis", basis),
                    ("workspace", workspace)):
        setattr(args, name, _ptr(t))
    args.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if events is not None:
        args.ev_main_begin, args.ev_main_end = events
    return args


def xkv_workspace_size(args):
    n = lib().lowram_xkv_workspace_size(ctypes.byref(args))
    if n == 0:
        raise LowramError(ERR_ARG, last_error() or "invalid arguments")
    return n


def xkv_launch(args, stream=None):
    rc = lib().lowram_xkv_factorize(ctypes.byref(args), _stream(stream))
    if rc != OK:
        raise LowramError(rc, last_error())


def xkv_factorize(keys, omega, n_iter=3, *, want_basis=False, workspace=None, stream=None):
    """Cross-layer key factors of Bt layer groups (keys [Bt, G, T, D], or one
    group [G, T, D]): returns a dict with a [Bt, T, r] bf16, b_l [Bt, G, D, r]
    bf16 and basis [Bt, G*D, r] float64 (when asked), without the batch
    dimension for a single group."""
    single = keys.dim() == 3
    k4 = keys.unsqueeze(0) if single else keys
    Bt, G, T, D = k4.shape
    r = omega.shape[1]
    dev = keys.device
    out = {"a": torch.empty(Bt, T, r, dtype=torch.bfloat16, device=dev),
           "b_l": torch.empty(Bt, G, D, r, dtype=torch.bfloat16, device=dev),
           "basis": torch.empty(Bt, G * D, r, dtype=torch.float64, device=dev) if want_basis else None}
    args = make_xkv_args(k4, omega, n_iter, out["a"], out["b_l"], basis=out["basis"])
    if workspace is None:
        workspace = torch.empty(xkv_workspace_size(args), dtype=torch.uint8, device=dev)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel()
    xkv_launch(args, stream)
    if single:
        out = {k: (None if v is None else v[0]) for k, v in out.items()}
    return out


def _run(fn, args, size_fn, device, workspace, stream):
    if workspace is None:
        n = size_fn(ctypes.byref(args))
        if n == 0:
            raise LowramError(ERR_ARG, last_error() or "invalid arguments")
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
    args.workspace = workspace.data_ptr()
    args.workspace_bytes = workspace.numel()
    rc = fn(ctypes.byref(args), _stream(stream))
    if rc != OK:
        raise LowramError(rc, last_error())


def pinv_value_map(w_k, w_v, *, want_f64=False, workspace=None, stream=None):
    """W_lin = pinv(W_K) W_V for P maps: w_k, w_v [P, hidden, d] bf16 ->
    (w_lin [P, d, d] bf16 output-major, w_lin64 float64 or None)."""
    P, hidden, d = w_k.shape
    args = PinvArgs()
    args.n_maps, args.hidden, args.head_dim = P, hidden, d
    w_lin = torch.empty(P, d, d, dtype=torch.bfloat16, device=w_k.device)
    w64 = torch.empty(P, d, d, dtype=torch.float64, device=w_k.device) if want_f64 else None
    for name, t in (("w_k", w_k), ("w_v", w_v), ("w_lin", w_lin), ("w_lin64", w64)):
        setattr(args, name, _ptr(t))
    L = lib()
    _run(L.lowram_pinv_value_map, args, L.lowram_pinv_workspace_size, w_k.device, workspace, stream)
    return w_lin, w64


def make_fit_args(keys, v, w_lin, w1, b1, w2, b2, n_steps, lr, *, losses=None, workspace=None, events=None):
    """Fill a FitArgs: keys [L, T, Hkv*d] bf16, v [L, T, Hkv, d] bf16,
    w_lin [L, Hkv, d, d] bf16, float32 parameters w1 [L, Hkv, h, d],
    b1 [L, Hkv, h], w2 [L, Hkv, d, h], b2 [L, Hkv, d] (updated in place)."""
    Lr, T, hkv, d = v.shape
    args = FitArgs()
    args.n_layers, args.ctx_len, args.n_kv_heads, args.head_dim = Lr, T, hkv, d
    args.mlp_hidden, args.n_steps, args.lr = w1.shape[2], n_steps, lr
    for name, t in (("keys", keys), ("v", v), ("w_lin", w_lin), ("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2),
                    ("losses", losses), ("workspace", workspace)):
        setattr(args, name, _ptr(t))
    args.workspace_bytes = 0 if workspace is None else workspace.numel()
    if events is not None:
        args.ev_main_begin, args.ev_main_end = events
    return args


def fit_workspace_size(args):
    n = lib().lowram_fit_workspace_size(ctypes.byref(args))
    if n == 0:
        raise LowramError(ERR_ARG, last_error() or "invalid arguments")
    return n


def fit_launch(args, stream=None):
    rc = lib().lowram_fit_predictor(ctypes.byref(args), _stream(stream))
    if rc != OK:
        raise LowramError(rc, last_error())


def fit_predictor(keys, v, w_lin, w1, b1, w2, b2, n_steps, lr, *, want_losses=True, workspace=None, stream=None):
    """n_steps of gradient descent on the nonlinear branch of every (layer, KV
    head) predictor; updates w1, b1, w2, b2 in place and returns the losses
    [L, Hkv, n_steps + 1] (None with want_losses=False, which also skips the
    loss-only pass after the last step)."""
    Lr, T, hkv, d = v.shape
    losses = torch.empty(Lr, hkv, n_steps + 1, dtype=torch.float32, device=v.device) if want_losses else None
    args = make_fit_args(keys, v, w_lin, w1, b1, w2, b2, n_steps, lr, losses=losses)
    L = lib()
    _run(L.lowram_fit_predictor, args, L.lowram_fit_workspace_size, v.device, workspace, stream)
    return losses
