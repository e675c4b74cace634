"""LowRAM decode-time path on MI355X (gfx950): reconstructed-KV attention over
a compressed cache, the prefill-side residual ranking, the cross-layer key
factorisation and the predictor's pseudoinverse start and test-time fit, as
HIP kernels behind the C ABI declared in include/lowram.h.
This package is the thin Python binding; build the library with
``python -m long_context_decode_lowram_amd.build``."""
from ._binding import (BF16, F32, FLAG_GENERIC, FLAG_VALIDATE, I2, I8, BLOCK, DecodeArgs, WindowArgs,
                       CHECK_SEL_ORDER, CHECK_RES_RANGE, CHECK_RES_ORDER, CHECK_RES_PTR, CHECK_WIN_LEN,
                       make_window_args, window_launch, window_append, decode_launch_noalloc, NOALLOC_SCRATCH_BYTES, LowramError, PrefillArgs, RankArgs,
                       XkvArgs, decode_launch, decode_step, decode_workspace_size, last_error, lib,
                       make_decode_args, make_prefill_args, make_rank_args, make_xkv_args, prefill_launch,
                       prefill_rank, prefill_workspace_size, rank_launch, rank_residuals, rank_workspace_size,
                       status_string, xkv_factorize, xkv_launch, xkv_workspace_size, PinvArgs, FitArgs,
                       pinv_value_map, make_fit_args, fit_workspace_size, fit_launch, fit_predictor)

__all__ = ["BF16", "F32", "FLAG_GENERIC", "FLAG_VALIDATE", "I2", "I8", "BLOCK", "DecodeArgs", "WindowArgs",
           "CHECK_SEL_ORDER", "CHECK_RES_RANGE", "CHECK_RES_ORDER", "CHECK_RES_PTR", "CHECK_WIN_LEN",
           "make_window_args", "window_launch", "window_append", "decode_launch_noalloc",
           "NOALLOC_SCRATCH_BYTES", "LowramError", "PrefillArgs", "RankArgs",
           "XkvArgs", "decode_launch", "decode_step", "decode_workspace_size", "last_error", "lib",
           "make_decode_args", "make_prefill_args", "make_rank_args", "make_xkv_args", "prefill_launch",
           "prefill_rank", "prefill_workspace_size", "rank_launch", "rank_residuals", "rank_workspace_size",
           "status_string", "xkv_factorize", "xkv_launch", "xkv_workspace_size", "PinvArgs", "FitArgs",
           "pinv_value_map", "make_fit_args", "fit_workspace_size", "fit_launch", "fit_predictor"]
