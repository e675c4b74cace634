"""Full-size GPU parity: each workload at its real shape and launch
configuration (the whole batch in one call, as the benchmark times it); the
float64 oracle checks sampled sequences one by one. Stats are exact."""
import numpy as np
import pytest
import torch

import synth
from _cases import TOL, gpu_decode, make_case, oracle_decode, rel_err

pytestmark = pytest.mark.gpu


def run(cfg, layer, samples, **kw):
    case = make_case(cfg, layer=layer, device="cuda", biases=False, **kw)
    out, stats = gpu_decode(case)
    for b in samples:
        ref, rstats = oracle_decode(case, batch_index=b)
        err = rel_err(out[b:b + 1].float().cpu().numpy(), ref)
        print(f"{cfg.name} layer {layer} b={b}: rel_err={err:.2e}", flush=True)
        assert err <= TOL[cfg.act]
        np.testing.assert_array_equal(stats[b:b + 1].cpu().numpy(), rstats)
    return case


def test_c2_mistral_group_all_layers():
    cfg = synth.CONFIGS["c2_mistral_group"]
    for layer in range(cfg.n_layers):
        run(cfg, layer, [0])


def test_c3_llama_131k_one_layer():
    cfg = synth.CONFIGS["c3_llama_131k"]
    run(cfg, 13, [0, 3])


def test_c4_llama_262k_batch8_with_window():
    cfg = synth.CONFIGS["c4_llama_262k"]
    run(cfg, 30, [0, 7], win_len=128)


def test_c5_composed_int8_evicted():
    cfg = synth.CONFIGS["c5_composed"]
    run(cfg, 5, [0, 11])
