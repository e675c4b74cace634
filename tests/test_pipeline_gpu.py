"""End to end on the tiny fp32 workload: the residual store comes from the
GPU ranking of the true values, and the decode runs on it.

True values (a reading of the workload's description): V = K W_lin +
gelu(K W1') W2' + noise, with (W1', W2') an independent draw of the
predictor's shapes and noise N(0, 0.05); the predictor sees (W_lin, W1, W2)
with W1 = W1', W2 = 0.9 W2', so it misses part of the nonlinear term and the
noise. The oracle builds K, V_hat and V in float64 (rounded to float32, the
storage dtype); both sides then rank the same tensors and decode the same
store."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _cases import np64, rel_err

pytestmark = pytest.mark.gpu

C1 = synth.CONFIGS["c1_tiny_f32"]


def true_and_predicted_values(layer):
    a, _ = synth.gen_group_factor(C1, layer // C1.group, "cpu")
    x = synth.gen_layer(C1, layer, "cpu")
    g = synth.make_generator("cpu", C1.seed, "truth", layer)
    w1t = torch.randn(C1.n_kv_heads, C1.mlp_hidden, 128, generator=g) / np.sqrt(128)
    w2t = torch.randn(C1.n_kv_heads, 128, C1.mlp_hidden, generator=g) / np.sqrt(128)
    noise = torch.randn(C1.ctx_len, C1.n_kv_heads, 128, generator=g) * 0.05
    x["w1"] = w1t.to(torch.float32)[None]
    x["w2"] = (0.9 * w2t).to(torch.float32)[None]
    keys = oracle.reconstruct_keys(np64(a[0]), np64(x["bl"][0]))
    v = np.zeros((1, C1.ctx_len, C1.n_kv_heads, 128))
    vh = np.zeros_like(v)
    for h in range(C1.n_kv_heads):
        k_h = keys[:, h * 128:(h + 1) * 128]
        vh[0, :, h] = oracle.predict_values(k_h, np64(x["w_lin"][0, h]), np64(x["w1"][0, h]), np64(x["w2"][0, h]))
        v[0, :, h] = (oracle.predict_values(k_h, np64(x["w_lin"][0, h]), np64(w1t[h]), np64(w2t[h]))
                      + np64(noise[:, h]))
    return a, x, v.astype(np.float32), vh.astype(np.float32)


def test_c1_rank_then_decode_four_layers():
    import long_context_decode_lowram_amd as L
    k = C1.n_res
    for layer in range(C1.n_layers):
        a, x, v, vh = true_and_predicted_values(layer)
        r = L.rank_residuals(torch.from_numpy(v).cuda(), torch.from_numpy(vh).cuda(), k, "f32")
        torch.cuda.synchronize()
        ro = oracle.rank_residuals(v, vh, k, 64, "f32")
        np.testing.assert_array_equal(r["idx"].cpu().numpy(), ro["idx"])
        np.testing.assert_array_equal(r["ptr"].cpu().numpy(), ro["ptr"])
        np.testing.assert_array_equal(r["val"].cpu().numpy().astype(np.float64), ro["val"])
        # Decode on the GPU store, oracle on its own store (identical, checked above).
        out = L.decode_step(x["q"].cuda(), a.cuda(), x["bl"].cuda(), x["w_lin"].cuda(), x["w1"].cuda(),
                            x["w2"].cuda(), r["idx"].cuda(), r["val"].cuda(), r["ptr"].cuda())
        torch.cuda.synchronize()
        ref, _ = oracle.decode_step(dict(q=np64(x["q"]), a=np64(a), bl=np64(x["bl"]), w_lin=np64(x["w_lin"]),
                                         w1=np64(x["w1"]), w2=np64(x["w2"]), res_idx=ro["idx"],
                                         res_val=ro["val"], block=64))
        err = rel_err(out.cpu().numpy(), ref)
        print(f"layer {layer}: rel_err={err:.2e}", flush=True)
        assert err <= 1e-4
