"""Decode-step benchmark: reconstructed-KV attention over the compressed cache.

One step = one decode token for every sequence in the batch: the layer
loop of lowram_decode_step calls over all layers of the workload (each call
rebuilds the selected blocks' keys, predicts values, adds residuals and runs
GQA attention), inputs resident in HBM. Prints one JSON line with the
cached-tokens/s metric of the headline workload (c3_llama_131k: batch 4,
131072 cached tokens, 32 layers), the fused kernel's roofline and the float64
oracle's rate on a bounded sample of the same workload. The same line holds,
under "legs", the other timed workloads, each with its own step time,
roofline and oracle sample:
  * c4_llama_262k_b8: batch 8, 262144 cached tokens, 32 layers, as the
    long-context protocol runs it: 128 consecutive decode steps, each with a
    fresh query and block selection per layer, appending the new token's
    exact key and value to every layer's recent-window buffer (1024 rows), so
    step s attends s + 1 window tokens; 2 warmup and 5 timed repeats of the
    128 steps;
  * c5_composed: batch 12, 131072 cached tokens, int8 factors and residuals,
    half the blocks evicted;
  * rank_residuals: the prefill-side ranking over 32 x 131072 x 8 (token,
    head) rows.

Timing of a decode workload: after the warmup steps, K eager steps run with
HIP events around every fused kernel (its average duration feeds the
roofline); then the step's calls are captured once into a HIP graph and K
replays of it are timed for ms_per_step and the metric (--no-graph times the
eager steps instead; eager_ms_per_step is reported either way).

python bench.py [--steps K] [--warmup W] [--workload c3_llama_131k] [--batch B] [--no-legs]
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_F32_VALU_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
METRIC = "decode-step reconstructed-KV attention: cached tokens/s and % of HBM roofline"
DECODE_SRC = os.path.join(ROOT, "long_context_decode_lowram_amd", "csrc", "decode_mfma.hip")
RANK_SRC = os.path.join(ROOT, "long_context_decode_lowram_amd", "csrc", "rank.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c3_llama_131k")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--generic", action="store_true", help="force the fp32 SIMT kernel")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step as eager launches instead of replays of a HIP graph of it")
    ap.add_argument("--overlap", action="store_true",
                    help="run each layer's combine on a second stream, beside the next layer's fused kernel")
    ap.add_argument("--res-dtype", choices=("f32", "bf16", "i8", "i2"), default=None,
                    help="store the workload's residuals in this encoding instead")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the headline's oracle sample")
    ap.add_argument("--leg-cpu-seconds", type=float, default=5.0, help="budget of each leg's oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="time the headline workload only")
    ap.add_argument("--legs", default="c4_llama_262k_b8,c5_composed,rank_residuals",
                    help="comma-separated legs to run after the headline")
    ap.add_argument("--leg", default=None, help="run this one leg alone (its object is the printed line)")
    ap.add_argument("--protocol", action="store_true",
                    help="time --workload with the 128-step window-append protocol (c4_llama_262k shapes)")
    ap.add_argument("--protocol-steps", type=int, default=128)
    ap.add_argument("--protocol-repeats", type=int, default=5)
    ap.add_argument("--protocol-warmups", type=int, default=2)
    ap.add_argument("--sweep", default=None,
                    help="with --protocol: comma-separated batch sizes, each timed in turn (OOM recorded)")
    ap.add_argument("--rank", action="store_true", help="also time the residual ranking at its full shape")
    ap.add_argument("--xkv", action="store_true", help="also time the cross-layer key factorisation")
    ap.add_argument("--fit", action="store_true", help="also time the predictor's test-time fit")
    ap.add_argument("--prefill", action="store_true",
                    help="also time the fused prefill ranking (V_hat computed in the library) at its full shape")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (reference dispatch for HBM byte counters)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]

    def create(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def create_sync(self):
        """An event for ordering only (hipEventDisableTiming)."""
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreateWithFlags(ctypes.byref(e), 2) == 0
        return e.value

    def record(self, e, stream):
        assert self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream.cuda_stream)) == 0

    def wait(self, stream, e):
        assert self.lib.hipStreamWaitEvent(ctypes.c_void_p(stream.cuda_stream), ctypes.c_void_p(e), 0) == 0

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return f.value

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


def attended_counts(inp, cfg, sel=None):
    """Per sequence: attended compressed tokens and residual rows that fall in
    attended blocks (exact, from the selection and the block CSR). ``sel``
    overrides the layer's own selection (a later step's)."""
    import torch
    sel = inp["sel"] if sel is None else sel
    B, nb = inp["res_ptr"].shape[0], cfg.nb
    mask = torch.zeros(B, nb, dtype=torch.bool, device=inp["res_ptr"].device)
    if sel is None:
        mask[:] = True
    else:
        valid = (sel >= 0) & (sel < nb)
        mask.scatter_(1, torch.where(valid, sel, 0).long(), valid)
    if inp["keep"] is not None:
        mask &= inp["keep"].bool()
    sizes = torch.full((nb,), cfg.block, device=mask.device)
    sizes[-1] = cfg.ctx_len - (nb - 1) * cfg.block
    n_att = (mask * sizes).sum(1)
    per_blk = (inp["res_ptr"][..., 1:] - inp["res_ptr"][..., :-1]).long()        # [B, Hkv, nb]
    n_res_att = (per_blk * mask[:, None, :]).sum((1, 2))
    return n_att.tolist(), n_res_att.tolist()


def work_per_call(cfg, n_att, n_res_att, win):
    """Algorithmic bytes and FLOPs of one layer call (all sequences).

    Bytes: every attended A row once (int8 rows add their scale), every
    residual row applied (value, index, int8 scale), the layer factor, the
    predictor, q and out, the window rows. FLOPs: key rebuild 2*r*Hkv*d,
    K W1 2*Hkv*d*h per token, scores 2*Hq*d and weighted sums 2*Hq*(d + h)
    per token (P [K | gelu]), and W_lin once per group of four blocks
    2*Hq*d*d: the linear parts W_lin, W2 and b2 are applied after the
    attention-weighted sum, an exact rewrite of the per-token predictor."""
    d, hkv, hq, r, h = cfg.head_dim, cfg.n_kv_heads, cfg.n_q_heads, cfg.rank, cfg.mlp_hidden
    ea = {"f32": 4, "bf16": 2, "i8": 1}[cfg.a_dtype]
    ew = {"f32": 4, "bf16": 2}[cfg.act]
    byts = flops = flops_direct = 0
    for na, nr in zip(n_att, n_res_att):
        byts += na * (r * ea + (4 if cfg.a_dtype == "i8" else 0))
        byts += nr * residual_row_bytes(cfg)
        byts += (r * hkv * d + hkv * (d * d + 2 * d * h)) * ew + 2 * hq * d * ew + win * 2 * hkv * d * ew
        flops += 2 * na * hkv * d * (r + h) + 2 * na * hq * d + 2 * na * hq * (d + h) + 2 * hq * d * d * -(-na // (4 * cfg.block))
        flops_direct += 2 * na * r * hkv * d + 2 * na * hkv * (d * d + 2 * d * h) + 4 * (na + win) * hq * d
    return byts, flops, flops_direct


def recorded_traffic(name, kernel_src, prefix="decode_mfma_kernel"):
    """HBM bytes per launch of a kernel from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE passes scaled by a calibration copy), or None
    when there is none for this workload or the kernel source has changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{prefix}_{name}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    text = open(path).read()
    if f"sha256 ({os.path.basename(kernel_src)}): {sha}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch="):
            return float(line.split("=", 1)[1])
    return None


def residual_row_bytes(cfg):
    """Bytes of one stored residual: the value row (2-bit codes pack four per
    byte), its int32 token index and, for int8 and 2-bit codes, a float32 scale."""
    d = cfg.head_dim
    row = {"f32": 4 * d, "bf16": 2 * d, "i8": d, "i2": d // 4}[cfg.res_dtype]
    return row + 4 + (4 if cfg.res_dtype in ("i8", "i2") else 0)


def stored_bytes(cfg):
    """Compressed cache bytes per sequence over all layers (factors, predictor,
    residuals with indices and block pointers) and the dense bf16 K+V bytes."""
    d, hkv, r, h, T = cfg.head_dim, cfg.n_kv_heads, cfg.rank, cfg.mlp_hidden, cfg.ctx_len
    ea = {"f32": 4, "bf16": 2, "i8": 1}[cfg.a_dtype]
    ew = {"f32": 4, "bf16": 2}[cfg.act]
    groups = -(-cfg.n_layers // cfg.group)
    a = groups * T * (r * ea + (4 if cfg.a_dtype == "i8" else 0))
    per_layer = r * hkv * d * ew + hkv * (d * d + 2 * d * h) * ew
    per_layer += hkv * cfg.n_res * residual_row_bytes(cfg) + hkv * (cfg.nb + 1) * 4
    stored = a + cfg.n_layers * per_layer
    dense = cfg.n_layers * 2 * hkv * d * 2 * T
    return stored, dense


def is_generic(cfg, forced):
    return forced or not (cfg.act == "bf16" and cfg.a_dtype in ("bf16", "i8")
                          and cfg.mlp_hidden % 64 == 0 and cfg.rank % 64 == 0)


def roofline(cfg, generic, launch_flops, launch_bytes, direct_flops, kern_avg_ms, name):
    achieved = launch_flops / (kern_avg_ms * 1e-3) / 1e12
    peak = PEAK_F32_VALU_TFLOPS if generic else PEAK_BF16_TFLOPS
    return {"bound": "alu" if generic else "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": None if generic else recorded_traffic(name, DECODE_SRC),
            "kernel": "decode_generic_kernel" if generic else "decode_mfma_kernel",
            "kernel_avg_ms": kern_avg_ms, "flops_per_launch": launch_flops, "bytes_per_launch": launch_bytes,
            "direct_method_flops_per_launch": direct_flops}


def config_json(cfg, name, generic, blocks, win):
    return {"workload": name, "batch": cfg.batch, "ctx_len": cfg.ctx_len, "layers": cfg.n_layers, "rank": cfg.rank,
            "mlp_hidden": cfg.mlp_hidden, "blocks_attended_per_layer": blocks, "n_res": cfg.n_res,
            "a_dtype": cfg.a_dtype, "res_dtype": cfg.res_dtype, "evicted_half": cfg.evict_half, "window": win,
            "kernel": "generic-f32" if generic else "mfma-bf16"}


def dtype_json(cfg):
    return "f32" if cfg.act == "f32" else ("bf16+i8" if cfg.a_dtype == "i8" else "bf16")


def run_decode(cfg, name, args, ev, *, steps, warmup, cpu_seconds, with_cpu):
    """The decode workload with a fixed window (the config's window rows, up to
    128): eager steps with events around every fused kernel, then graph
    replays of the step. Returns the result dict."""
    import torch
    import long_context_decode_lowram_amd as L
    import synth

    dev = "cuda"
    t0 = time.time()
    groups = [synth.gen_group_factor(cfg, g, dev) for g in range(-(-cfg.n_layers // cfg.group))]
    layers = [synth.gen_layer(cfg, l, dev) for l in range(cfg.n_layers)]
    win = min(cfg.win_cap, 128) if cfg.win_cap else 0
    wins = [synth.gen_window(cfg, l, dev) if cfg.win_cap else (None, None) for l in range(cfg.n_layers)]
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    print(f"# generated {name} B={cfg.batch} in {gen_s:.1f}s, "
          f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB resident", file=sys.stderr, flush=True)

    outs = [torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=layers[0]["q"].dtype, device=dev)
            for _ in range(cfg.n_layers)]
    calls = []
    for l, x in enumerate(layers):
        a, a_scale = groups[l // cfg.group]
        wk, wv = wins[l]
        calls.append(L.make_decode_args(x["q"], a, x["bl"], x["w_lin"], x["w1"], x["w2"], x["res_idx"],
                                        x["res_val"], x["res_ptr"], outs[l], a_scale=a_scale, b1=x["b1"],
                                        b2=x["b2"], res_scale=x["res_scale"], sel=x["sel"], keep=x["keep"],
                                        win_k=wk, win_v=wv, win_len=win, generic=args.generic))
    ws_bytes = max(L.decode_workspace_size(c) for c in calls)
    # Two workspaces, alternating by layer: each layer's combine runs on a
    # second stream and overlaps the next layer's fused kernel, which writes
    # the other workspace; layer l+2 waits for layer l's combine.
    overlap = args.overlap
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(2 if overlap else 1)]
    for l, c in enumerate(calls):
        c.workspace, c.workspace_bytes = wss[l % len(wss)].data_ptr(), ws_bytes

    counts = [attended_counts(x, cfg) for x in layers]
    step_bytes = step_flops = step_flops_direct = 0
    for n_att, n_res_att in counts:
        b_, f_, fd_ = work_per_call(cfg, n_att, n_res_att, win)
        step_bytes, step_flops, step_flops_direct = step_bytes + b_, step_flops + f_, step_flops_direct + fd_

    stream = torch.cuda.current_stream()
    n_ev = steps * cfg.n_layers
    evs = [(ev.create(), ev.create()) for _ in range(n_ev)]
    cstream = torch.cuda.Stream() if overlap else None
    ready = [ev.create_sync() for _ in calls] if overlap else []
    done = [ev.create_sync() for _ in calls] if overlap else []
    for l, c in enumerate(calls):
        if overlap:
            c.combine_stream, c.combine_ready = cstream.cuda_stream, ready[l]

    def step(timed_index=None, s=None):
        ms_ = stream if s is None else s
        for l, c in enumerate(calls):
            if timed_index is not None:
                c.ev_main_begin, c.ev_main_end = evs[timed_index * cfg.n_layers + l]
            else:
                c.ev_main_begin = c.ev_main_end = None
            if overlap and l >= 2:
                ev.wait(ms_, done[l - 2])            # layer l-2's combine has released this workspace
            L.decode_launch(c, ms_)
            if overlap:
                ev.record(done[l], cstream)
        if overlap:
            for l in range(max(0, len(calls) - 2), len(calls)):
                ev.wait(ms_, done[l])                # join: the step ends with every combine

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Eager timed region: every fused kernel bracketed by HIP events on its
    # stream (the roofline's kernel duration).
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(stop) / steps
    ms = eager_ms
    timing = "eager launches"
    if not args.no_graph:
        # Graph timed region: the step's layer calls captured once into a HIP
        # graph (the entry point only enqueues kernels) and replayed, which
        # removes the host launch gaps between them. Should capture fail, the
        # eager timing stands and the line says why.
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step(s=torch.cuda.current_stream())
            for _ in range(max(1, warmup)):
                graph.replay()
            torch.cuda.synchronize()
            start.record(stream)
            for i in range(steps):
                graph.replay()
            stop.record(stream)
            torch.cuda.synchronize()
            ms = start.elapsed_time(stop) / steps
            timing = "HIP graph replays of the step"
        except RuntimeError as exc:
            torch.cuda.synchronize()
            timing = f"eager launches (graph capture failed: {exc})"
    kernel_ms = [ev.elapsed_ms(a, b) for a, b in evs]
    kern_avg_ms = sum(kernel_ms) / len(kernel_ms)
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)

    generic = is_generic(cfg, args.generic)
    cached = cfg.batch * (cfg.ctx_len + win)
    hbm_gbs = step_bytes / (ms * 1e-3) / 1e9
    stored, dense = stored_bytes(cfg)
    blocks = int(sum(c[0][0] for c in counts) / cfg.n_layers // cfg.block)
    result = {
        "metric": METRIC, "value": cached / (ms * 1e-3), "unit": "cached tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": ms,
        "timing": timing + ("; each layer's combine overlaps the next layer's fused kernel" if overlap else ""),
        "eager_ms_per_step": eager_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype_json(cfg),
        "data": "synthetic (seeded draws at Llama-3.1-8B / Mistral-7B attention shapes)",
        "config": config_json(cfg, name, generic, blocks, win),
        "hbm": {"algorithmic_bytes_per_step": step_bytes, "achieved_GBs": hbm_gbs,
                "frac_of_8TBs": hbm_gbs / PEAK_HBM_GBS},
        "roofline": roofline(cfg, generic, step_flops / cfg.n_layers, step_bytes / cfg.n_layers,
                             step_flops_direct / cfg.n_layers, kern_avg_ms, name),
        "attention_only_decode_tokens_per_s": cfg.batch / (ms * 1e-3),
        "compression_ratio": dense / stored,
        "input_generation_s": gen_s,
    }
    if with_cpu:
        result["cpu_baseline"], result["parity"] = cpu_baseline(cfg, groups, layers, wins, outs, win, cpu_seconds)
    return result


def run_protocol(cfg, name, args, ev, *, n_steps, repeats, warmups, cpu_seconds, with_cpu):
    """The long-context protocol: n_steps consecutive decode steps, each with
    the step's query and block selection staged for every layer (plain device
    copies from draws made beforehand), the new token's exact key and value
    appended to every layer's window buffer by lowram_window_append, and the
    layer calls reading their window length from the device count the append
    advanced; step s attends s + 1 window tokens. The append and the layer
    calls are captured once into a HIP graph, replayed once per step. One
    eager pass with events around every fused kernel gives the kernel
    average. Returns the result dict, or {"oom": ...} when the inputs do not
    fit in device memory."""
    import torch
    import long_context_decode_lowram_amd as L
    import synth

    dev = "cuda"
    nl, bsz, width, cap = cfg.n_layers, cfg.batch, cfg.n_kv_heads * cfg.head_dim, cfg.win_cap
    t0 = time.time()
    try:
        groups = [synth.gen_group_factor(cfg, g, dev) for g in range(-(-nl // cfg.group))]
        layers = [synth.gen_layer(cfg, l, dev) for l in range(nl)]
        act = layers[0]["q"].dtype
        win_k = torch.zeros(nl, bsz, cap, width, dtype=act, device=dev)
        win_v = torch.zeros_like(win_k)
        draws = [synth.gen_step_inputs(cfg, s, dev) for s in range(n_steps)]
        q_all = torch.stack([d_["q"] for d_ in draws])
        sel_all = None if draws[0]["sel"] is None else torch.stack([d_["sel"] for d_ in draws])
        nk_all = torch.stack([d_["new_k"] for d_ in draws])
        nv_all = torch.stack([d_["new_v"] for d_ in draws])
        del draws
        torch.cuda.synchronize()
    except torch.OutOfMemoryError as exc:
        groups = layers = win_k = win_v = None
        torch.cuda.empty_cache()
        return {"oom": str(exc).splitlines()[0], "config": {"workload": name, "batch": bsz}}
    gen_s = time.time() - t0
    print(f"# generated {name} B={bsz} ({n_steps} steps of draws) in {gen_s:.1f}s, "
          f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB resident", file=sys.stderr, flush=True)

    count = torch.zeros(nl, dtype=torch.int32, device=dev)
    q_st, nk_st, nv_st = q_all[0].clone(), nk_all[0].clone(), nv_all[0].clone()
    sel_st = None if sel_all is None else sel_all[0].clone()
    outs = [torch.empty(bsz, cfg.n_q_heads, cfg.head_dim, dtype=act, device=dev) for _ in range(nl)]
    calls = []
    for l, x in enumerate(layers):
        a, a_scale = groups[l // cfg.group]
        calls.append(L.make_decode_args(q_st[l], a, x["bl"], x["w_lin"], x["w1"], x["w2"], x["res_idx"],
                                        x["res_val"], x["res_ptr"], outs[l], a_scale=a_scale, b1=x["b1"],
                                        b2=x["b2"], res_scale=x["res_scale"],
                                        sel=None if sel_st is None else sel_st[l], keep=x["keep"],
                                        win_k=win_k[l], win_v=win_v[l], win_len=cap,
                                        win_len_dev=count[l:l + 1], generic=args.generic))
    ws_bytes = max(L.decode_workspace_size(c) for c in calls)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    for c in calls:
        c.workspace, c.workspace_bytes = ws.data_ptr(), ws_bytes
    wargs = L.make_window_args(nk_st, nv_st, win_k, win_v, count)
    stream = torch.cuda.current_stream()

    def stage(s):
        q_st.copy_(q_all[s])
        if sel_st is not None:
            sel_st.copy_(sel_all[s])
        nk_st.copy_(nk_all[s])
        nv_st.copy_(nv_all[s])

    def launch(st, events=None):
        L.window_launch(wargs, st)
        for l, c in enumerate(calls):
            c.ev_main_begin, c.ev_main_end = (None, None) if events is None else events[l]
            L.decode_launch(c, st)

    # Algorithmic work of every (step, layer) call, from that step's selection.
    step_bytes = step_flops = step_flops_direct = 0.0
    for s in range(n_steps):
        for l, x in enumerate(layers):
            n_att, n_res_att = attended_counts(x, cfg, None if sel_all is None else sel_all[s, l])
            b_, f_, fd_ = work_per_call(cfg, n_att, n_res_att, s + 1)
            step_bytes, step_flops, step_flops_direct = step_bytes + b_, step_flops + f_, step_flops_direct + fd_
    step_bytes, step_flops, step_flops_direct = (x_ / n_steps for x_ in (step_bytes, step_flops, step_flops_direct))

    # One eager pass of the protocol with events around every fused kernel.
    evs = [[(ev.create(), ev.create()) for _ in range(nl)] for _ in range(n_steps)]
    count.zero_()
    for s in range(n_steps):
        stage(s)
        launch(stream, evs[s])
    torch.cuda.synchronize()
    kernel_ms = [ev.elapsed_ms(a, b) for row in evs for a, b in row]
    kern_avg_ms = sum(kernel_ms) / len(kernel_ms)
    for row in evs:
        for a, b in row:
            ev.destroy(a)
            ev.destroy(b)
    for c in calls:
        c.ev_main_begin = c.ev_main_end = None

    count.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch(torch.cuda.current_stream())
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rep_ms = []
    for r in range(warmups + repeats):
        count.zero_()
        start.record(stream)
        for s in range(n_steps):
            stage(s)
            graph.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        if r >= warmups:
            rep_ms.append(start.elapsed_time(stop) / n_steps)
    assert count.tolist() == [min(n_steps, cap)] * nl
    ms = sorted(rep_ms)[len(rep_ms) // 2]

    generic = is_generic(cfg, args.generic)
    mean_win = sum(min(s + 1, cap) for s in range(n_steps)) / n_steps
    cached = bsz * (cfg.ctx_len + mean_win)
    hbm_gbs = step_bytes / (ms * 1e-3) / 1e9
    stored, dense = stored_bytes(cfg)
    n_sel_blocks = cfg.n_sel if sel_all is not None else cfg.nb
    result = {
        "metric": METRIC, "value": cached / (ms * 1e-3), "unit": "cached tokens/s", "n_gpus": 1,
        "ms_per_step": ms, "repeat_ms_per_step": rep_ms,
        "protocol": f"{n_steps} consecutive decode steps per repeat, {warmups} warmup and {repeats} timed repeats "
                    f"(median reported); each step stages that step's query and block selection for every layer, "
                    f"appends the new token's exact key and value to every layer's window (lowram_window_append) and "
                    f"runs the {nl} layer calls, which read the window length from the device count: step s attends "
                    f"s + 1 window tokens (capacity {cap}); append and layer calls replayed as one HIP graph per step",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype_json(cfg),
        "data": "synthetic (seeded draws at Llama-3.1-8B attention shapes)",
        "config": config_json(cfg, name, generic, n_sel_blocks, f"1..{min(n_steps, cap)} (mean {mean_win:g})"),
        "hbm": {"algorithmic_bytes_per_step": step_bytes, "achieved_GBs": hbm_gbs,
                "frac_of_8TBs": hbm_gbs / PEAK_HBM_GBS},
        "roofline": roofline(cfg, generic, step_flops / nl, step_bytes / nl, step_flops_direct / nl, kern_avg_ms,
                             name),
        "attention_only_decode_tokens_per_s": bsz / (ms * 1e-3),
        "compression_ratio": dense / stored,
        "input_generation_s": gen_s,
    }
    if with_cpu:
        last = n_steps - 1
        lay = [dict(x, q=q_all[last, l], sel=None if sel_all is None else sel_all[last, l])
               for l, x in enumerate(layers)]
        wins = [(win_k[l], win_v[l]) for l in range(nl)]
        result["cpu_baseline"], result["parity"] = cpu_baseline(cfg, groups, lay, wins, outs, min(n_steps, cap),
                                                                cpu_seconds)
        result["parity"]["step"] = last
    return result


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported "
                          "(the path shards by sequence; one GPU is what this library times)"}))
        sys.exit(2)
    import torch
    import synth

    cfg = synth.CONFIGS[args.workload]
    if args.res_dtype is not None:
        cfg = cfg.replace(res_dtype=args.res_dtype)
    if args.batch:
        cfg = cfg.replace(batch=args.batch)
    torch.cuda.init()
    ev = HipEvents()
    with_cpu = not args.no_cpu_baseline

    if args.protocol:
        batches = [int(b) for b in args.sweep.split(",")] if args.sweep else [cfg.batch]
        sweep = []
        for bsz in batches:
            r = run_protocol(cfg.replace(batch=bsz), args.workload, args, ev, n_steps=args.protocol_steps,
                             repeats=args.protocol_repeats, warmups=args.protocol_warmups,
                             cpu_seconds=args.cpu_seconds, with_cpu=with_cpu and bsz == batches[0])
            torch.cuda.empty_cache()
            print(f"# {args.workload} B={bsz}: " + (f"{r['ms_per_step']:.3f} ms/step, {r['value']:.4g} cached tok/s"
                                                   if "oom" not in r else "out of memory"), file=sys.stderr, flush=True)
            sweep.append(r)
        result = sweep[0] if len(sweep) == 1 else dict(sweep[-1] if "oom" not in sweep[-1] else sweep[0],
                                                       sweep=sweep)
        result.update(steps=args.protocol_steps * args.protocol_repeats, warmup=args.protocol_steps * args.protocol_warmups)
        print(json.dumps(result), flush=True)
        return

    def run_leg(leg, cpu_seconds):
        t0 = time.time()
        if leg == "c4_llama_262k_b8":
            c4 = synth.CONFIGS["c4_llama_262k"]
            r = run_protocol(c4, "c4_llama_262k_b8", args, ev, n_steps=args.protocol_steps,
                             repeats=args.protocol_repeats, warmups=args.protocol_warmups,
                             cpu_seconds=cpu_seconds, with_cpu=with_cpu)
        elif leg == "c5_composed":
            r = run_decode(synth.CONFIGS["c5_composed"], leg, args, ev, steps=5, warmup=2,
                           cpu_seconds=cpu_seconds, with_cpu=with_cpu)
        elif leg == "rank_residuals":
            r = bench_rank(args.steps, args.warmup, ev, cpu_seconds=cpu_seconds, with_cpu=with_cpu)
        else:
            raise SystemExit(f"unknown leg {leg}")
        r["leg_wall_s"] = time.time() - t0
        torch.cuda.empty_cache()
        print(f"# leg {leg}: {r['leg_wall_s']:.1f}s", file=sys.stderr, flush=True)
        return r

    if args.leg:
        result = run_leg(args.leg, args.cpu_seconds)
        if args.calibrate_copy:
            calibration_copy(result)
        print(json.dumps(result), flush=True)
        return
    result = run_decode(cfg, args.workload, args, ev, steps=args.steps, warmup=args.warmup,
                        cpu_seconds=args.cpu_seconds, with_cpu=with_cpu)
    torch.cuda.empty_cache()
    if not args.no_legs and args.workload == "c3_llama_131k" and not args.generic:
        result["legs"] = {leg: run_leg(leg, args.leg_cpu_seconds) for leg in args.legs.split(",") if leg}
    if args.rank and not (result.get("legs") or {}).get("rank_residuals"):
        result["rank_residuals"] = bench_rank(args.steps, args.warmup, ev, cpu_seconds=args.leg_cpu_seconds,
                                              with_cpu=False)
    if args.prefill:
        result["prefill_rank"] = bench_prefill(max(2, args.steps // 3), 1, ev)
    if args.xkv:
        result["xkv_factorize"] = bench_xkv(max(2, args.steps // 3), 1, ev)
    if args.fit:
        result["fit_predictor"] = bench_fit(2, 1, ev)
    if args.calibrate_copy:
        calibration_copy(result)
    print(json.dumps(result), flush=True)


def calibration_copy(result):
    """A plain 1 GiB device copy: the reference dispatch that scales the HBM
    byte counters (FETCH_SIZE, WRITE_SIZE) of a profiled run."""
    import torch
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    result["calibration_copy_bytes"] = 1 << 30


def cpu_baseline(cfg, groups, layers, wins, outs, win, budget_s):
    """The float64 oracle on sequence 0 of successive layers (until the time
    budget is spent), timed on this host's cores, and the relative error of
    the GPU outputs of those same (sequence, layer) pairs against it."""
    import numpy as np
    import threadpoolctl
    import torch
    import oracle

    def host(t):
        if t is None:
            return None
        t = t[0:1]
        return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()

    layer_s, errs, used = [], [], 0
    with threadpoolctl.threadpool_limits(limits=len(os.sched_getaffinity(0))):
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        for l in range(cfg.n_layers):
            a, a_scale = groups[l // cfg.group]
            x = layers[l]
            batch = {k: host(x[k]) for k in ("q", "bl", "w_lin", "w1", "w2", "b1", "b2", "res_idx", "res_val",
                                             "res_scale", "sel", "keep")}
            batch.update(a=host(a), a_scale=host(a_scale), block=cfg.block, win_len=win,
                         win_k=host(wins[l][0]), win_v=host(wins[l][1]))
            t0 = time.time()
            ref, _ = oracle.decode_step(batch)
            layer_s.append(time.time() - t0)
            got = outs[l][0:1].float().cpu().numpy()
            errs.append(float(np.max(np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1))))
            used += 1
            if sum(layer_s) >= budget_s:
                break
    t_layer = sum(layer_s) / len(layer_s)
    rate = (cfg.ctx_len + win) / (cfg.n_layers * t_layer)
    return ({"value": rate, "unit": "cached tokens/s", "cores": threads, "kind": "oracle",
             "sample": f"sequence 0 of layers 0..{used - 1} ({used} of {cfg.n_layers} layer calls, "
                       f"{sum(layer_s):.1f} s); step rate extrapolated as one sequence x all layers",
             "seconds_per_layer_call": t_layer},
            {"oracle_layers_checked": used, "max_rel_err": max(errs), "tolerance": 2e-2 if cfg.act == "bf16" else 1e-4})


def bench_rank(steps, warmup, ev, *, cpu_seconds=5.0, with_cpu=True):
    """lowram_rank_residuals at the composed workload's ranking shape: 32
    slices x 131072 tokens x 8 KV heads, bf16 V and V_hat, k = 13107, int8
    residuals. The error kernel (every row of V and V_hat read once, one
    binary64 error written per row) is timed by HIP events on its stream and
    carries the roofline against HBM; the whole call's rate is ranked
    (token, head) rows per second. The oracle ranks whole slices (all heads)
    on the host for the CPU baseline and the parity sample."""
    import numpy as np
    import torch
    import long_context_decode_lowram_amd as L
    import synth

    rc = synth.RANK_C5
    v, vh = synth.gen_rank_inputs(rc, "cuda", plant_ties=False)
    Lr, T, hkv, d = v.shape
    k, nb = rc.n_res, -(-T // 64)
    o = {"idx": torch.empty(Lr, hkv, k, dtype=torch.int32, device="cuda"),
         "val": torch.empty(Lr, hkv, k, d, dtype=torch.int8, device="cuda"),
         "scale": torch.empty(Lr, hkv, k, dtype=torch.float32, device="cuda"),
         "ptr": torch.empty(Lr, hkv, nb + 1, dtype=torch.int32, device="cuda")}
    args = L.make_rank_args(v, vh, k, "i8", o["idx"], o["val"], o["scale"], o["ptr"])
    ws = torch.empty(L.rank_workspace_size(args), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    for _ in range(warmup):
        L.rank_launch(args)
    torch.cuda.synchronize()
    evs = [(ev.create(), ev.create()) for _ in range(steps)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(steps):
        args.ev_main_begin, args.ev_main_end = evs[i]
        L.rank_launch(args)
    s1.record()
    torch.cuda.synchronize()
    args.ev_main_begin = args.ev_main_end = None
    ms = s0.elapsed_time(s1) / steps
    err_ms = sum(ev.elapsed_ms(a, b) for a, b in evs) / steps
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    in_bytes = 2 * v.numel() * v.element_size()
    err_bytes = in_bytes + Lr * hkv * T * 8
    achieved = err_bytes / (err_ms * 1e-3) / 1e9
    rows = Lr * T * hkv
    result = {"metric": "residual ranking: ranked (token, head) rows/s", "value": rows / (ms * 1e-3),
              "unit": "ranked rows/s", "ms_per_call": ms, "steps": steps, "warmup": warmup,
              "config": {"workload": "c5_rank", "shape": [Lr, T, hkv, d], "n_res": k, "in_dtype": "bf16",
                         "res_dtype": "i8"},
              "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": achieved / PEAK_HBM_GBS,
                           "traffic": recorded_traffic("c5_rank", RANK_SRC, prefix="rank_error_kernel"),
                           "kernel": "rank_error_kernel", "kernel_avg_ms": err_ms, "bytes_per_launch": err_bytes},
              "whole_call_input_GBs": in_bytes / (ms * 1e-3) / 1e9}
    if with_cpu:
        import threadpoolctl
        import oracle
        with threadpoolctl.threadpool_limits(limits=len(os.sched_getaffinity(0))):
            info = threadpoolctl.threadpool_info()
            threads = max([i.get("num_threads", 1) for i in info] or [1])
            used, t_cpu, exact = 0, 0.0, True
            while used < Lr and (used == 0 or t_cpu < cpu_seconds):
                sl = used
                hv = v[sl:sl + 1].float().cpu().numpy()
                hh = vh[sl:sl + 1].float().cpu().numpy()
                t0 = time.time()
                ref = oracle.rank_residuals(hv, hh, k, 64, "i8")
                t_cpu += time.time() - t0
                exact &= bool(np.array_equal(o["idx"][sl:sl + 1].cpu().numpy(), ref["idx"])
                              and np.array_equal(o["ptr"][sl:sl + 1].cpu().numpy(), ref["ptr"])
                              and np.array_equal(o["val"][sl:sl + 1].cpu().numpy(), ref["val"]))
                used += 1
        result["cpu_baseline"] = {"value": used * T * hkv / t_cpu, "unit": "ranked rows/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"slices 0..{used - 1} of {Lr} (all {hkv} heads each, {t_cpu:.1f} s)"}
        result["parity"] = {"oracle_slices_checked": used, "index_exact": exact}
    return result


def bench_prefill(steps, warmup, ev):
    """The fused prefill ranking at the composed workload's ranking shape:
    32 layers of 131072 tokens, 8 KV heads, r = 512, h = 256, k = 13107,
    int8 residuals. The all-token pass is timed by HIP events on the stream
    it runs on; its work is the MFMA products of every token and head."""
    import torch
    import long_context_decode_lowram_amd as L
    import synth

    pc = synth.PREFILL_CONFIGS["p_c5"]
    x = synth.gen_prefill_inputs(pc, "cuda")
    Lr, T, hkv, d = x["v"].shape
    k, nb, r, h = pc.n_res, -(-T // 64), pc.rank, pc.hidden
    o = {"idx": torch.empty(Lr, hkv, k, dtype=torch.int32, device="cuda"),
         "val": torch.empty(Lr, hkv, k, d, dtype=torch.int8, device="cuda"),
         "scale": torch.empty(Lr, hkv, k, dtype=torch.float32, device="cuda"),
         "ptr": torch.empty(Lr, hkv, nb + 1, dtype=torch.int32, device="cuda")}
    args = L.make_prefill_args(x["a"], x["b_l"], x["w_lin"], x["w1"], x["w2"], x["v"], k, "i8", o["idx"],
                               o["val"], o["scale"], o["ptr"], group=pc.group)
    ws = torch.empty(L.prefill_workspace_size(args), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    for _ in range(warmup):
        L.prefill_launch(args)
    torch.cuda.synchronize()
    evs = [(ev.create(), ev.create()) for _ in range(steps)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(steps):
        args.ev_main_begin, args.ev_main_end = evs[i]
        L.prefill_launch(args)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / steps
    pass1_ms = sum(ev.elapsed_ms(a, b) for a, b in evs) / steps
    flops = 2.0 * d * (r + d + 2 * h) * T * hkv * Lr
    return {"shape": [Lr, T, hkv, d], "rank": r, "mlp_hidden": h, "n_res": k, "ms_per_call": ms,
            "all_token_pass_ms": pass1_ms, "all_token_pass_TFLOPs": flops / (pass1_ms * 1e-3) / 1e12,
            "all_token_pass_frac_of_bf16_peak": flops / (pass1_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "v_read_GBs": x["v"].numel() * 2 / (ms * 1e-3) / 1e9}


def bench_xkv(steps, warmup, ev):
    """The cross-layer key factorisation of a whole Llama-3.1-8B prefill at
    131072 tokens: 32 layers in 8 groups of 4 (8 KV heads x 128 per layer),
    rank 512, 3 iterations, all 8 groups in one call. The Gram kernel (bf16
    MFMA over every token) is timed by HIP events on the stream it runs on;
    its work is the T n (n + 1) flops of the symmetric product's unique
    entries."""
    import torch
    import long_context_decode_lowram_amd as L
    import synth

    xc = synth.XKV_CONFIGS["x_llama_131k"]
    bt = 8
    x = synth.gen_xkv_inputs(xc, "cuda", batch=bt)
    T, n, r = xc.ctx_len, xc.n, xc.rank
    o = {"a": torch.empty(bt, T, r, dtype=torch.bfloat16, device="cuda"),
         "b_l": torch.empty(bt, xc.n_layers, xc.width, r, dtype=torch.bfloat16, device="cuda")}
    args = L.make_xkv_args(x["keys"], x["omega"], xc.n_iter, o["a"], o["b_l"])
    ws = torch.empty(L.xkv_workspace_size(args), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    for _ in range(warmup):
        L.xkv_launch(args)
    torch.cuda.synchronize()
    evs = [(ev.create(), ev.create()) for _ in range(steps)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(steps):
        args.ev_main_begin, args.ev_main_end = evs[i]
        L.xkv_launch(args)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / steps
    gram_ms = sum(ev.elapsed_ms(a, b) for a, b in evs) / steps
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    gram_flops = float(T) * n * (n + 1) * bt
    return {"groups": bt, "layers_per_group": xc.n_layers, "ctx_len": T, "width": xc.width, "rank": r,
            "n_iter": xc.n_iter, "ms_per_call": ms, "ms_per_group": ms / bt,
            "keys_GBs": x["keys"].numel() * 2 / (ms * 1e-3) / 1e9, "gram_kernel_ms": gram_ms,
            "gram_kernel_TFLOPs": gram_flops / (gram_ms * 1e-3) / 1e12,
            "gram_kernel_frac_of_bf16_peak": gram_flops / (gram_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_fit(steps, warmup, ev):
    """The predictor's test-time fit for a whole Llama-3.1-8B prefill at
    131072 tokens: 32 layers x 8 KV heads, h = 256, the quick two-step fit,
    all (layer, head) problems in one call. The gradient steps are timed by
    HIP events on the stream they run on; their work is 2 d (5 h + d) FLOP per
    token and problem (forward W1 and W_lin/W2 products, the W2 product of the
    backward, and the two weight-gradient products)."""
    import torch
    import long_context_decode_lowram_amd as L
    import synth

    fc = synth.FIT_CONFIGS["f_llama_131k"]
    x = synth.gen_fit_inputs(fc, "cuda")
    P, T, d, h = fc.n_layers * fc.n_kv_heads, fc.ctx_len, fc.head_dim, fc.hidden
    losses = torch.empty(fc.n_layers, fc.n_kv_heads, fc.n_steps + 1, dtype=torch.float32, device="cuda")
    args = L.make_fit_args(x["keys"], x["v"], x["w_lin"], x["w1"], x["b1"], x["w2"], x["b2"], fc.n_steps, fc.lr,
                           losses=losses)
    ws = torch.empty(L.fit_workspace_size(args), dtype=torch.uint8, device="cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    for _ in range(warmup):
        L.fit_launch(args)
    torch.cuda.synchronize()
    evs = [(ev.create(), ev.create()) for _ in range(steps)]
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(steps):
        args.ev_main_begin, args.ev_main_end = evs[i]
        L.fit_launch(args)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / steps
    step_ms = sum(ev.elapsed_ms(a, b) for a, b in evs) / steps / fc.n_steps
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    flops = 2.0 * d * (5 * h + d) * T * P
    return {"problems": P, "ctx_len": T, "hidden": h, "n_steps": fc.n_steps, "lr": fc.lr, "ms_per_call": ms,
            "ms_per_gradient_step": step_ms, "step_TFLOPs": flops / (step_ms * 1e-3) / 1e12,
            "step_frac_of_bf16_peak": flops / (step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "loss_first_last_mean": [float(losses[..., 0].mean()), float(losses[..., -1].mean())]}


if __name__ == "__main__":
    main()
