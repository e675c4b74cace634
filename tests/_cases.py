"""Helpers shared by the GPU parity tests: build a seeded case, run it through
the C ABI and through the float64 oracle, and compare."""
import numpy as np
import torch

import oracle
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def np64(t):
    if t is None:
        return None
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()


def make_case(cfg, layer=0, *, device="cpu", biases=True, q_scale=1.0, win_len=0, batch=None):
    bsz = cfg.batch if batch is None else batch
    a, a_scale = synth.gen_group_factor(cfg, layer // cfg.group, device, batch=bsz)
    case = synth.gen_layer(cfg, layer, device, biases=biases, q_scale=q_scale, batch=bsz)
    case.update(a=a, a_scale=a_scale, win_len=win_len, win_k=None, win_v=None)
    if cfg.win_cap:
        case["win_k"], case["win_v"] = synth.gen_window(cfg, layer, device, batch=bsz)
    return case


def set_residuals(case, cfg, idx):
    """Replace the residual set with explicit ascending indices [B, Hkv, k]."""
    bsz, hkv = idx.shape[:2]
    k = idx.shape[-1]
    g = synth.make_generator("cpu", cfg.seed, "set_res", k)
    dev = case["q"].device
    case["res_idx"] = idx.to(torch.int32).to(dev).contiguous()
    if cfg.res_dtype == "i8":
        case["res_val"] = torch.randint(-127, 128, (bsz, hkv, k, 128), generator=g).to(torch.int8).to(dev)
        case["res_scale"] = (torch.rand(bsz, hkv, k, generator=g) * 1e-3 + 1e-4).to(dev)
    elif cfg.res_dtype == "i2":
        case["res_val"] = torch.randint(0, 256, (bsz, hkv, k, 32), generator=g, dtype=torch.int32).to(torch.uint8).to(dev)
        case["res_scale"] = (torch.rand(bsz, hkv, k, generator=g) * 0.05 + 0.01).to(dev)
    else:
        dt = torch.float32 if cfg.res_dtype == "f32" else torch.bfloat16
        case["res_val"] = (torch.randn(bsz, hkv, k, 128, generator=g) * 0.05).to(dt).to(dev)
        case["res_scale"] = None
    case["res_ptr"] = synth.block_ptr_from_idx(case["res_idx"], cfg.ctx_len, cfg.block)
    return case


def to(case, device):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in case.items()}


def gpu_decode(case, *, generic=False, with_stats=True, out=None):
    import long_context_decode_lowram_amd as L
    c = to(case, "cuda")
    q = c["q"]
    stats = torch.full((q.shape[0], c["bl"].shape[1] // 128, 2), -7, dtype=torch.int32, device="cuda") \
        if with_stats else None
    out = L.decode_step(c["q"], c["a"], c["bl"], c["w_lin"], c["w1"], c["w2"], c["res_idx"], c["res_val"],
                        c["res_ptr"], out=out, a_scale=c["a_scale"], b1=c["b1"], b2=c["b2"],
                        res_scale=c["res_scale"], sel=c["sel"], keep=c["keep"], win_k=c["win_k"],
                        win_v=c["win_v"], win_len=c["win_len"], stats=stats, generic=generic)
    torch.cuda.synchronize()
    return out, stats


def oracle_decode(case, batch_index=None):
    names = ["q", "a", "a_scale", "bl", "w_lin", "w1", "b1", "w2", "b2", "res_idx", "res_val", "res_scale",
             "sel", "keep", "win_k", "win_v"]
    sl = slice(None) if batch_index is None else slice(batch_index, batch_index + 1)
    batch = {n: (None if case.get(n) is None else np64(case[n][sl])) for n in names}
    batch["block"] = 64
    batch["win_len"] = case["win_len"]
    return oracle.decode_step(batch)


def rel_err(got, ref):
    """Max over rows of ||got - ref||_2 / ||ref||_2 (rows with a zero
    reference must match exactly)."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "rows with a zero reference must be zero"
    return float(np.max(num[~zero] / den[~zero])) if (~zero).any() else 0.0


class WindowSession:
    """A few decode steps of every layer, the way the long-context protocol
    runs them: per step the query and block selection of each layer are
    staged, lowram_window_append writes the new token's exact key and value
    into each layer's window buffer and advances its device count, and each
    layer's lowram_decode_step reads its window length from that count.
    Group factors are generated once per group and shared by its layers."""

    def __init__(self, cfg, cap, *, biases=True):
        import long_context_decode_lowram_amd as L
        self.L, self.cfg, self.cap = L, cfg, cap
        nl, bsz, w = cfg.n_layers, cfg.batch, cfg.n_kv_heads * cfg.head_dim
        act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
        groups = [synth.gen_group_factor(cfg, g, "cuda") for g in range(-(-nl // cfg.group))]
        self.cases = []
        for l in range(nl):
            c = synth.gen_layer(cfg, l, "cuda", biases=biases)
            a, a_scale = groups[l // cfg.group]
            c.update(a=a, a_scale=a_scale, win_len=0, win_k=None, win_v=None)
            self.cases.append(c)
        self.win_k = torch.zeros(nl, bsz, cap, w, dtype=act, device="cuda")
        self.win_v = torch.zeros_like(self.win_k)
        self.count = torch.zeros(nl, dtype=torch.int32, device="cuda")
        st = synth.gen_step_inputs(cfg, 0, "cuda")
        self.q = torch.empty_like(st["q"])
        self.sel = None if st["sel"] is None else torch.empty_like(st["sel"])
        self.new_k, self.new_v = torch.empty_like(st["new_k"]), torch.empty_like(st["new_v"])
        self.outs = [torch.empty_like(c["q"]) for c in self.cases]
        self.stats = [torch.empty(bsz, cfg.n_kv_heads, 2, dtype=torch.int32, device="cuda") for _ in self.cases]
        self.calls = []
        for l, c in enumerate(self.cases):
            self.calls.append(L.make_decode_args(
                self.q[l], c["a"], c["bl"], c["w_lin"], c["w1"], c["w2"], c["res_idx"], c["res_val"], c["res_ptr"],
                self.outs[l], a_scale=c["a_scale"], b1=c["b1"], b2=c["b2"], res_scale=c["res_scale"],
                sel=None if self.sel is None else self.sel[l], keep=c["keep"], win_k=self.win_k[l],
                win_v=self.win_v[l], win_len=cap, win_len_dev=self.count[l:l + 1], stats=self.stats[l]))
        ws = max(L.decode_workspace_size(a) for a in self.calls)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        for a in self.calls:
            a.workspace, a.workspace_bytes = self.ws.data_ptr(), ws
        self.wargs = L.make_window_args(self.new_k, self.new_v, self.win_k, self.win_v, self.count)

    def stage(self, step):
        st = synth.gen_step_inputs(self.cfg, step, "cuda")
        self.q.copy_(st["q"])
        if self.sel is not None:
            self.sel.copy_(st["sel"])
        self.new_k.copy_(st["new_k"])
        self.new_v.copy_(st["new_v"])
        return st

    def launch(self, stream=None):
        self.L.window_launch(self.wargs, stream)
        for a in self.calls:
            self.L.decode_launch(a, stream)

    def oracle(self, l, n_win, st, batch_index=None):
        c = dict(self.cases[l])
        c.update(q=st["q"][l], sel=None if st["sel"] is None else st["sel"][l], win_k=self.win_k[l],
                 win_v=self.win_v[l], win_len=n_win)
        return oracle_decode(c, batch_index)
