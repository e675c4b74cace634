"""Seeded synthetic inputs for the decode step and the residual ranking.

This module draws inputs only: it holds none of the method's arithmetic (no
key rebuild, no predictor, no softmax, no error ranking, no quantiser). Both
the HIP path and the float64 oracle consume what it produces; neither imports
the other. Tensors are produced with torch on the requested device (CPU for
small cases, the GPU for full-size workloads) from generators seeded by a hash
of (config seed, tensor name, layer, step); bf16 and int8 tensors are drawn
in their storage dtype, so the oracle reads the same values by exact upcast.

Shapes follow the workloads: Mistral-7B and Llama-3.1-8B attention shapes
(32 query / 8 KV heads, head_dim 128, 32 layers in groups of 4), block 64.
No dataset items are used; the pages' benchmarks (LongBench, RULER) are stood
in for by these draws.
"""
import dataclasses
import hashlib
import math

import torch

__all__ = ["DecodeConfig", "CONFIGS", "RankConfig", "RANK_C5", "PrefillConfig", "PREFILL_CONFIGS",
           "make_generator", "n_blocks", "gen_group_factor", "gen_layer", "gen_window", "gen_step_inputs",
           "gen_rank_inputs",
           "gen_prefill_inputs", "block_ptr_from_idx", "XkvConfig", "XKV_CONFIGS", "gen_xkv_inputs",
           "FitConfig", "FIT_CONFIGS", "gen_fit_inputs", "gen_pinv_inputs"]


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    ctx_len: int
    n_layers: int
    rank: int
    mlp_hidden: int
    res_frac: tuple            # (num, den): k = floor(T*num/den)
    sel_den: int               # 1 = every block, else n_sel = nb / sel_den
    act: str                   # 'f32' | 'bf16'  (q, factors, weights, window, out)
    a_dtype: str               # 'f32' | 'bf16' | 'i8'
    res_dtype: str             # 'f32' | 'bf16' | 'i8' | 'i2'
    evict_half: bool = False
    win_cap: int = 0
    steps: int = 1
    group: int = 4
    n_q_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    block: int = 64
    seed: int = 0

    @property
    def n_res(self):
        num, den = self.res_frac
        return (self.ctx_len * num) // den

    @property
    def nb(self):
        return -(-self.ctx_len // self.block)

    @property
    def n_sel(self):
        return self.nb // self.sel_den

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c1_tiny_f32": DecodeConfig("c1_tiny_f32", 1, 4096, 4, 256, 64, (1, 5), 1, "f32", "f32", "f32", seed=1),
    "c2_mistral_group": DecodeConfig("c2_mistral_group", 1, 32768, 4, 512, 256, (1, 5), 4, "bf16", "bf16",
                                     "bf16", seed=2),
    "c3_llama_131k": DecodeConfig("c3_llama_131k", 4, 131072, 32, 1024, 256, (1, 5), 8, "bf16", "bf16",
                                  "bf16", seed=3),
    "c4_llama_262k": DecodeConfig("c4_llama_262k", 8, 262144, 32, 1024, 256, (1, 5), 16, "bf16", "bf16",
                                  "bf16", win_cap=1024, steps=128, seed=4),
    "c5_composed": DecodeConfig("c5_composed", 12, 131072, 32, 512, 256, (1, 10), 1, "bf16", "i8", "i8",
                                evict_half=True, seed=5),
}


@dataclasses.dataclass(frozen=True)
class RankConfig:
    n_slices: int
    ctx_len: int
    n_kv_heads: int = 8
    head_dim: int = 128
    block: int = 64
    res_frac: tuple = (1, 10)
    in_dtype: str = "bf16"
    res_dtype: str = "i8"
    seed: int = 5

    @property
    def n_res(self):
        num, den = self.res_frac
        return (self.ctx_len * num) // den


RANK_C5 = RankConfig(32, 131072)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    """Shapes of the fused prefill ranking: Lr layers in groups sharing a key
    factor, their per-layer key factor and predictor, and the true values."""
    name: str
    n_slices: int
    ctx_len: int
    rank: int
    hidden: int
    n_res: int
    n_kv_heads: int = 8
    group: int = 4
    head_dim: int = 128
    block: int = 64
    res_dtype: str = "i8"
    biases: bool = False
    seed: int = 6


PREFILL_CONFIGS = {c.name: c for c in (
    PrefillConfig("p_small_ragged", 4, 1000, 256, 128, 100, n_kv_heads=2, res_dtype="bf16", biases=True),
    PrefillConfig("p_mid", 8, 8192, 512, 256, 819),
    # the composed workload's ranking shape (32 layers of 131072 tokens, Mistral-7B attention
    # shapes, r = 512, h = 256, k = floor(0.1 T))
    PrefillConfig("p_c5", 32, 131072, 512, 256, 13107),
)}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
_SIGMA = 1.0 / math.sqrt(128.0)     # N(0, 1/sqrt(d)) draws, d = 128


def n_blocks(ctx_len, block):
    return -(-ctx_len // block)


def make_generator(device, *key):
    """A torch generator on ``device`` seeded by a hash of ``key``."""
    h = hashlib.blake2b(repr(key).encode(), digest_size=8).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h, "little") & ((1 << 63) - 1))
    return g


def _normal(shape, std, dtype, device, g):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (x * std).to(dtype)


def _int8_rows(shape, std, device, g):
    """int8 codes with a float32 scale per row, drawn directly (codes from a
    rounded normal of std 40, scales around std/40)."""
    codes = torch.randn(shape, generator=g, device=device).mul_(40.0).round_().clamp_(-127, 127)
    scale = torch.rand(shape[:-1], generator=g, device=device).add_(0.5).mul_(std / 40.0)
    return codes.to(torch.int8), scale.to(torch.float32)


def _i2_rows(shape, std, device, g):
    """2-bit codes packed four per byte ([..., d/4] uint8, every byte value
    equally likely) with a float32 scale per row around std / 1.118 (the rms
    of the levels -1.5, -0.5, 0.5, 1.5 is 1.118)."""
    packed = torch.randint(0, 256, shape[:-1] + (shape[-1] // 4,), generator=g, device=device,
                           dtype=torch.int32)
    scale = torch.rand(shape[:-1], generator=g, device=device).add_(0.5).mul_(std / 1.118)
    return packed.to(torch.uint8), scale.to(torch.float32)


def gen_group_factor(cfg, group, device, batch=None):
    """The shared key factor A of one layer group: [B, T, r] in ``cfg.a_dtype``
    (int8 codes plus a [B, T] float32 scale for 'i8')."""
    bsz = cfg.batch if batch is None else batch
    g = make_generator(device, cfg.seed, "A", group)
    shape = (bsz, cfg.ctx_len, cfg.rank)
    if cfg.a_dtype == "i8":
        return _int8_rows(shape, _SIGMA, device, g)
    return _normal(shape, _SIGMA, _DT[cfg.a_dtype], device, g), None


def _selection(cfg, bsz, layer, step, device):
    """Per sequence: blocks {0, 1, nb-2, nb-1} plus n_sel-4 drawn uniformly
    without replacement from [2, nb-3], ascending (int32 [B, n_sel]). Below
    n_sel = 4 (tiny test contexts only) the rows keep the four edge blocks and
    come out longer than n_sel; callers take the row length from the tensor."""
    nb, n_sel = cfg.nb, cfg.n_sel
    g = make_generator("cpu", cfg.seed, "sel", layer, step)
    rows = []
    for _ in range(bsz):
        mid = torch.randperm(nb - 4, generator=g)[: n_sel - 4] + 2
        rows.append(torch.sort(torch.cat([torch.tensor([0, 1, nb - 2, nb - 1]), mid])).values)
    return torch.stack(rows).to(torch.int32).to(device)


def _keep_mask(cfg, bsz, layer, step, device):
    """Per sequence: exactly nb/2 blocks evicted, drawn from [2, nb-3] (uint8
    [B, nb], 1 = kept)."""
    nb = cfg.nb
    g = make_generator("cpu", cfg.seed, "keep", layer, step)
    keep = torch.ones(bsz, nb, dtype=torch.uint8)
    for b in range(bsz):
        ev = torch.randperm(nb - 4, generator=g)[: nb // 2] + 2
        keep[b, ev] = 0
    return keep.to(device)


def block_ptr_from_idx(idx, ctx_len, block):
    """Block CSR of ascending residual indices [..., k] -> [..., nb+1] int32
    (format conversion: ptr[i] = number of indices below i*block)."""
    nb = n_blocks(ctx_len, block)
    bounds = torch.arange(nb + 1, device=idx.device, dtype=idx.dtype) * block
    bounds[-1] = ctx_len
    rows = math.prod(idx.shape[:-1])
    flat = idx.reshape(rows, idx.shape[-1]).contiguous()
    ptr = torch.searchsorted(flat, bounds.expand(rows, nb + 1).contiguous())
    return ptr.reshape(*idx.shape[:-1], nb + 1).to(torch.int32)


def gen_residual_positions(cfg, bsz, layer, device):
    """Seeded uniform k-subsets of [0, T) per (b, KV head), ascending int32."""
    g = make_generator(device, cfg.seed, "res_idx", layer)
    k = cfg.n_res
    keys = torch.rand(bsz * cfg.n_kv_heads, cfg.ctx_len, generator=g, device=device)
    idx = torch.topk(keys, k, dim=1, sorted=False).indices
    idx = torch.sort(idx, dim=1).values.to(torch.int32)
    return idx.reshape(bsz, cfg.n_kv_heads, k)


def gen_layer(cfg, layer, device, *, step=0, batch=None, biases=False, res_idx=None,
              q_scale=1.0):
    """Everything one layer's decode call reads except the group factor.

    Returns a dict of tensors: q [B,Hq,d]; bl [B,Hkv*d,r] (B_l stored
    output-major); w_lin [B,Hkv,d,d]; w1 [B,Hkv,h,d]; w2 [B,Hkv,d,h];
    b1 [B,Hkv,h] and b2 [B,Hkv,d] when ``biases``; res_idx [B,Hkv,k] int32
    ascending; res_val [B,Hkv,k,d] (+ res_scale [B,Hkv,k] for 'i8');
    res_ptr [B,Hkv,nb+1] int32; sel [B,n_sel] int32 or None; keep [B,nb]
    uint8 or None. ``res_idx`` may be given (e.g. from a ranking run).
    ``q_scale`` rescales the query (the peaked-attention variant).
    """
    bsz = cfg.batch if batch is None else batch
    act = _DT[cfg.act]
    d, hkv, hq, r, h = cfg.head_dim, cfg.n_kv_heads, cfg.n_q_heads, cfg.rank, cfg.mlp_hidden
    g = make_generator(device, cfg.seed, "layer", layer, step)
    out = {
        "q": (torch.randn(bsz, hq, d, generator=g, device=device) * (_SIGMA * q_scale)).to(act),
        "bl": _normal((bsz, hkv * d, r), _SIGMA, act, device, g),
        "w_lin": _normal((bsz, hkv, d, d), _SIGMA, act, device, g),
        "w1": _normal((bsz, hkv, h, d), _SIGMA, act, device, g),
        "w2": _normal((bsz, hkv, d, h), _SIGMA, act, device, g),
        "b1": _normal((bsz, hkv, h), 0.05, act, device, g) if biases else None,
        "b2": _normal((bsz, hkv, d), 0.05, act, device, g) if biases else None,
    }
    if res_idx is None:
        res_idx = gen_residual_positions(cfg, bsz, layer, device)
    k = res_idx.shape[-1]
    gr = make_generator(device, cfg.seed, "res_val", layer)
    if cfg.res_dtype == "i8":
        out["res_val"], out["res_scale"] = _int8_rows((bsz, hkv, k, d), 0.05, device, gr)
    elif cfg.res_dtype == "i2":
        out["res_val"], out["res_scale"] = _i2_rows((bsz, hkv, k, d), 0.05, device, gr)
    else:
        out["res_val"] = _normal((bsz, hkv, k, d), 0.05, _DT[cfg.res_dtype], device, gr)
        out["res_scale"] = None
    out["res_idx"] = res_idx.to(device)
    out["res_ptr"] = block_ptr_from_idx(out["res_idx"], cfg.ctx_len, cfg.block)
    out["sel"] = None if cfg.sel_den == 1 else _selection(cfg, bsz, layer, step, device)
    out["keep"] = _keep_mask(cfg, bsz, layer, step, device) if cfg.evict_half else None
    return out


def gen_window(cfg, layer, device, *, batch=None):
    """Recent-window buffers [B, cap, Hkv*d] in the activation dtype. The kernel
    takes window tokens as given exact keys and values, so they are drawn
    i.i.d. (keys with std 0.25, the spread of the rebuilt keys under the
    factor draws; values with std 0.1)."""
    bsz = cfg.batch if batch is None else batch
    act = _DT[cfg.act]
    g = make_generator(device, cfg.seed, "win", layer)
    shape = (bsz, cfg.win_cap, cfg.n_kv_heads * cfg.head_dim)
    return _normal(shape, 0.25, act, device, g), _normal(shape, 0.1, act, device, g)


def gen_step_inputs(cfg, step, device, *, batch=None, n_layers=None):
    """What changes from one decode step to the next, for every layer: the
    query q [L, B, Hq, d], the block selection sel [L, B, n_sel] (None when
    every block is attended) and the new token's exact key and value rows
    new_k, new_v [L, B, Hkv*d], appended to the recent window (drawn like the
    window rows: keys with std 0.25, values with std 0.1). Keyed by step, so
    step s of a run always sees the same draws."""
    bsz = cfg.batch if batch is None else batch
    nl = cfg.n_layers if n_layers is None else n_layers
    act = _DT[cfg.act]
    g = make_generator(device, cfg.seed, "step", step, bsz, nl)
    width = cfg.n_kv_heads * cfg.head_dim
    q = (torch.randn(nl, bsz, cfg.n_q_heads, cfg.head_dim, generator=g, device=device) * _SIGMA).to(act)
    new_k = _normal((nl, bsz, width), 0.25, act, device, g)
    new_v = _normal((nl, bsz, width), 0.1, act, device, g)
    sel = None
    if cfg.sel_den != 1:
        sel = torch.stack([_selection(cfg, bsz, layer, step + 1, device) for layer in range(nl)])
    return {"q": q, "sel": sel, "new_k": new_k, "new_v": new_v}


def gen_rank_inputs(rc, device, *, n_slices=None, plant_ties=True):
    """Prefill-side ranking inputs V, V_hat [Lr, T, Hkv, d] in ``rc.in_dtype``.

    V_hat ~ N(0, 0.125); V = V_hat + eps * s with eps ~ N(0, 0.05) per element
    and s ~ LogNormal(0, 1) per (token, head), so a minority of tokens carry
    most of the error. With ``plant_ties``, per (slice, head): 1% of tokens
    copy another token's (V, V_hat) row exactly (equal errors at random
    places), k-2 tokens get a deviation 1e4 times larger (a top tier) and a
    group of 6 tokens share one identical row with a deviation 1e3 times
    larger, so that group straddles the k-th place.
    """
    ns = rc.n_slices if n_slices is None else n_slices
    dt = _DT[rc.in_dtype]
    T, hkv, d = rc.ctx_len, rc.n_kv_heads, rc.head_dim
    g = make_generator(device, rc.seed, "rank", ns, T)
    v_hat = (torch.randn(ns, T, hkv, d, generator=g, device=device) * 0.125).to(dt)
    s = torch.exp(torch.randn(ns, T, hkv, 1, generator=g, device=device))
    v = (v_hat.float() + torch.randn(ns, T, hkv, d, generator=g, device=device) * 0.05 * s).to(dt)
    if plant_ties:
        k = rc.n_res
        gc = make_generator("cpu", rc.seed, "rank-ties", ns, T)
        for sl in range(ns):
            for h in range(hkv):
                perm = torch.randperm(T, generator=gc)
                n_dup = max(1, T // 100)
                src, dst = perm[:n_dup], perm[n_dup:2 * n_dup]
                src, dst = src.to(device), dst.to(device)
                v[sl, dst, h] = v[sl, src, h]
                v_hat[sl, dst, h] = v_hat[sl, src, h]
                if k >= 2:
                    top = perm[2 * n_dup:2 * n_dup + k - 2].to(device)
                    v[sl, top, h] = (v_hat[sl, top, h].float() + 500.0 *
                                     torch.randn(top.numel(), d, generator=g, device=device).abs().add(0.5)).to(dt)
                grp = perm[2 * n_dup + max(k - 2, 0):2 * n_dup + max(k - 2, 0) + 6].to(device)
                if grp.numel():
                    v_hat[sl, grp, h] = v_hat[sl, grp[:1], h]
                    v[sl, grp, h] = (v_hat[sl, grp[:1], h].float() + 50.0).to(dt)
    return v.contiguous(), v_hat.contiguous()


def gen_prefill_inputs(pc, device, *, res_dtype=None):
    """Inputs of the fused prefill ranking, bf16: a [ceil(Lr/group), T, r],
    b_l [Lr, Hkv*d, r], w_lin [Lr, Hkv, d, d], w1 [Lr, Hkv, h, d],
    w2 [Lr, Hkv, d, h] (all N(0, 1/sqrt(128)), w2 N(0, 1/sqrt(h))), biases
    N(0, 0.05) when ``pc.biases``, and true values V [Lr, T, Hkv, d] drawn
    independently: N(0, 0.125) times a LogNormal(0, 1) scale per (token, head),
    so a minority of tokens carries large errors whatever the predictor gives.
    """
    g = make_generator(device, pc.seed, "prefill", pc.name)
    bf = torch.bfloat16
    ng = -(-pc.n_slices // pc.group)
    L, T, hkv, d, r, h = pc.n_slices, pc.ctx_len, pc.n_kv_heads, pc.head_dim, pc.rank, pc.hidden
    out = {
        "a": (torch.randn(ng, T, r, generator=g, device=device) * _SIGMA).to(bf),
        "b_l": (torch.randn(L, hkv * d, r, generator=g, device=device) * _SIGMA).to(bf),
        "w_lin": (torch.randn(L, hkv, d, d, generator=g, device=device) * _SIGMA).to(bf),
        "w1": (torch.randn(L, hkv, h, d, generator=g, device=device) * _SIGMA).to(bf),
        "w2": (torch.randn(L, hkv, d, h, generator=g, device=device) / math.sqrt(h)).to(bf),
        "b1": (torch.randn(L, hkv, h, generator=g, device=device) * 0.05).to(bf) if pc.biases else None,
        "b2": (torch.randn(L, hkv, d, generator=g, device=device) * 0.05).to(bf) if pc.biases else None,
    }
    s = torch.exp(torch.randn(L, T, hkv, 1, generator=g, device=device))
    out["v"] = (torch.randn(L, T, hkv, d, generator=g, device=device) * 0.125 * s).to(bf)
    return out


@dataclasses.dataclass(frozen=True)
class XkvConfig:
    """A layer group's keys for the cross-layer factorisation: G layers of
    [T, D] keys (D = Hkv d), factored at rank r with n_iter iterations. The
    concatenated keys are Z diag(s) W with Z [T, m] standard normal,
    s_i = exp(-i / decay) + floor and W [m, G D] normal / sqrt(m): energy in
    few directions with a slowly decaying tail, no gap at r."""
    name: str
    n_layers: int
    ctx_len: int
    width: int
    rank: int
    latent: int
    decay: float
    floor: float = 0.03
    n_iter: int = 3
    seed: int = 7

    @property
    def n(self):
        return self.n_layers * self.width


XKV_CONFIGS = {c.name: c for c in (
    XkvConfig("x_small_ragged", 2, 1000, 256, 64, 384, 40.0),
    XkvConfig("x_short", 2, 40, 256, 64, 64, 10.0),          # fewer tokens than the rank
    XkvConfig("x_mid", 4, 8192, 1024, 512, 1536, 200.0),
    XkvConfig("x_rank_max", 2, 3000, 1024, 1024, 1536, 300.0),  # the largest rank, ragged tokens
    # one group of four Llama-3.1-8B layers (8 KV heads x 128) at 131072 tokens, r = 512
    XkvConfig("x_llama_131k", 4, 131072, 1024, 512, 1536, 200.0),
)}


def gen_xkv_inputs(xc, device, batch=None):
    """keys [G, T, D] bf16 (scaled to unit rms), or [batch, G, T, D] with an
    independent draw per problem, and omega [G D, r] float64 standard normal,
    the iteration's starting block shared by the problems."""
    def one(tag):
        g = make_generator(device, xc.seed, "xkv", xc.name, tag)
        m = xc.latent
        s = torch.exp(-torch.arange(m, device=device, dtype=torch.float32) / xc.decay) + xc.floor
        z = torch.randn(xc.ctx_len, m, generator=g, device=device) * s
        w = torch.randn(m, xc.n, generator=g, device=device) / math.sqrt(m)
        cat = z @ w
        del z
        cat = cat / cat.pow(2).mean().sqrt()
        return cat.reshape(xc.ctx_len, xc.n_layers, xc.width).permute(1, 0, 2).contiguous().to(torch.bfloat16)
    keys = one(0) if batch is None else torch.stack([one(b) for b in range(batch)])
    g = make_generator(device, xc.seed, "xkv-omega", xc.name)
    omega = torch.randn(xc.n, xc.rank, generator=g, device=device, dtype=torch.float64)
    return {"keys": keys, "omega": omega}


@dataclasses.dataclass(frozen=True)
class FitConfig:
    """The predictor fit: L layers x Hkv heads of T tokens, hidden width h,
    n_steps of gradient descent at rate lr."""
    name: str
    n_layers: int
    ctx_len: int
    n_kv_heads: int
    hidden: int
    n_steps: int
    lr: float = 0.05
    head_dim: int = 128
    seed: int = 8


FIT_CONFIGS = {c.name: c for c in (
    FitConfig("f_small_ragged", 2, 1000, 2, 128, 3),
    FitConfig("f_mid", 2, 8192, 8, 256, 2, lr=0.02),
    # a hidden layer too wide for the resident-weight forward (the tiled one runs), ragged T
    FitConfig("f_wide_ragged", 1, 700, 2, 384, 2, lr=0.01),
    # a 32-layer Llama-3.1-8B prefill at 131072 tokens, h = 256, the quick two-step fit
    FitConfig("f_llama_131k", 32, 131072, 8, 256, 2, lr=0.02),
)}


def gen_fit_inputs(fc, device):
    """keys [L, T, Hkv*d] bf16 standard normal; w_lin [L, Hkv, d, d] bf16
    N(0, 1/sqrt(d)); true values v = k W_lin + gelu(k A) B + N(0, 0.05) with a
    hidden branch A [d, h] ~ N(0, 1/sqrt(d)), B [h, d] ~ N(0, 1/sqrt(h)) per
    head, so there is a nonlinear part to learn; the branch to fit starts at
    w1 ~ N(0, 1/sqrt(d)), b1 = 0, w2 = 0, b2 = 0 (float32), so the predictor
    starts at the linear map."""
    g = make_generator(device, fc.seed, "fit", fc.name)
    L, T, hkv, d, h = fc.n_layers, fc.ctx_len, fc.n_kv_heads, fc.head_dim, fc.hidden
    keys = torch.empty(L, T, hkv * d, dtype=torch.bfloat16, device=device)
    v = torch.empty(L, T, hkv, d, dtype=torch.bfloat16, device=device)
    w_lin = (torch.randn(L, hkv, d, d, generator=g, device=device) / math.sqrt(d)).to(torch.bfloat16)
    for l in range(L):
        k = torch.randn(T, hkv * d, generator=g, device=device).to(torch.bfloat16)
        keys[l] = k
        kf = k.float().view(T, hkv, d)
        for hh in range(hkv):
            a = torch.randn(d, h, generator=g, device=device) / math.sqrt(d)
            b = torch.randn(h, d, generator=g, device=device) / math.sqrt(h)
            x = kf[:, hh, :].contiguous()
            out = x @ w_lin[l, hh].float().t().contiguous() + torch.nn.functional.gelu(x @ a) @ b
            out += 0.05 * torch.randn(T, d, generator=g, device=device)
            v[l, :, hh, :] = out.to(torch.bfloat16)
    w1 = torch.randn(L, hkv, h, d, generator=g, device=device) / math.sqrt(d)
    return {"keys": keys, "v": v, "w_lin": w_lin, "w1": w1, "b1": torch.zeros(L, hkv, h, device=device),
            "w2": torch.zeros(L, hkv, d, h, device=device), "b2": torch.zeros(L, hkv, d, device=device)}


def gen_pinv_inputs(n_maps, hidden, device, seed=9, d=128):
    """W_K, W_V [P, hidden, d] bf16 with N(0, 1/sqrt(hidden)) entries."""
    g = make_generator(device, seed, "pinv", n_maps, hidden)
    w_k = (torch.randn(n_maps, hidden, d, generator=g, device=device) / math.sqrt(hidden)).to(torch.bfloat16)
    w_v = (torch.randn(n_maps, hidden, d, generator=g, device=device) / math.sqrt(hidden)).to(torch.bfloat16)
    return w_k, w_v
