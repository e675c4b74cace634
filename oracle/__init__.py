"""Float64 CPU oracle for LowRAM's decode-time path and its residual ranking.

TEST INFRASTRUCTURE ONLY. Nothing in the product package may import, call or
link this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
path (no kernels, headers, helpers or constants) and imports nothing from it.

Every function is the plain definition written out in numpy/scipy float64.
Inputs arrive in their storage dtype and are upcast exactly to float64 at the
point of use. Library primitives (matmul, SVD, pinv, erf, lexsort) serve as
single steps; there is no blocking, fusion or reordering beyond the definition.

Sources, cited by page title and the part of the page:
  * explainer   -- "LowRAM KV cache compression -- Predicting the value cache
                   from keys" (learnaivisually): the mechanism paragraph (keys
                   kept, per-head two-layer predictor fitted at prefill, exact
                   residuals for the worst tokens, values rebuilt as prediction
                   plus residual and fed to ordinary attention); the Slim
                   Attention paragraph (pseudoinverse start, exact recovery for
                   a square invertible key projection, GQA); the three-details
                   paragraph (head-specific map, error-ranked residuals); the
                   keys paragraph (xKV low-rank basis shared by adjacent
                   layers); the memory worked example; the prefill/decode cost
                   paragraph (selected chunks rebuilt at decode, new tokens
                   stored exactly).
  * project site -- "LowRAM -- Low-rank keys and amortised values for
                   composable KV cache compression at test time": Figure 1
                   (what the cache stores), Figure 3 (K ~ A.B, shared factor
                   per layer group, own factor per layer).
  * paper page  -- "LowRAM: Low-Rank Keys and Amortised Values for Composable
                   KV Cache Compression at Test-Time" (arXiv 2611.07025),
                   Abstract (residuals for the worst-reconstructed tokens;
                   only a selected subset of KV pairs rebuilt per step).
  * NovaKV card -- "Mistral-7B-NovaKV", Results table (dense cache per token).

Pins (tests/test_oracle_pins.py) tie every function to something other than
itself: the Slim Attention exact-recovery case, exact values when every token
has a residual, exact keys at full rank plus the Eckart-Young tail, a
pure-Python brute force on tiny inputs, ranking brute force and its special
cases, GELU identities, bf16/int8 rounding against library routines and closed
forms, and the explainer's printed memory arithmetic.
"""
from .decode import (gelu, reconstruct_keys, predict_values, attended_blocks,
                     decode_batch_element, decode_step, attention)
from .rank import (residual_error, select_worst, round_bf16, round_f32,
                   quantize_int8_rows, dequantize_int8_rows, quantize_i2_rows,
                   dequantize_i2_rows, pack_i2, unpack_i2, block_ptr, rank_residuals)
from .factor import xkv_factorize, xkv_subspace_iteration, pinv_value_map
from .fit import gelu_grad, predictor_loss_and_grads, fit_predictor
from .prefill import predicted_values, prefill_rank
from .budget import value_budget, dense_kv_bytes_per_token

__all__ = [
    "gelu", "reconstruct_keys", "predict_values", "attended_blocks",
    "decode_batch_element", "decode_step", "attention",
    "residual_error", "select_worst", "round_bf16", "round_f32",
    "quantize_int8_rows", "dequantize_int8_rows", "quantize_i2_rows", "dequantize_i2_rows",
    "pack_i2", "unpack_i2", "block_ptr", "rank_residuals",
    "xkv_factorize", "xkv_subspace_iteration", "pinv_value_map", "gelu_grad", "predictor_loss_and_grads",
    "fit_predictor", "value_budget", "dense_kv_bytes_per_token",
    "predicted_values", "prefill_rank",
]
