"""MI355X (gfx950) BLASST block-skipping attention.

A thin Python binding over the C ABI of ``libblasst.so`` (declared in
``include/blasst.h``).  Every function here only marshals arguments: torch
tensors are passed as device pointers, strides and element types, and every
step of the attention runs in the library's HIP kernels.  There is no CPU
fallback: if the library is missing, importing a call raises.

Entry points (same names as the C ABI):
  blasst_prefill(q, k, v, causal, lam, tile_q, ...)   -> O
  blasst_prefill_gaps(q, k, v, ...)                    -> gap map (calibration pass, no O)
  blasst_decode(q, k_cache, v_cache, seq_lens, lam, ...) -> O
  blasst_decode_gaps(q, k_cache, v_cache, seq_lens, ...) -> gap map (calibration pass, no O)
  blasst_decode_plan(...)                              -> (num_splits, workspace bytes)
  blasst_decode_noalloc(q, k_cache, v_cache, seq_lens, lam, ...) -> O (no workspace)
  blasst_decode_paged(q, k_pages, v_pages, page_table, seq_lens, Lmax, ...) -> O
  blasst_decode_paged_plan(...)                        -> (num_splits, workspace bytes)
  blasst_calibrate(table, target, L, tile_q=, block_k=, num_splits=) -> lambda = a(target) / L
  calib_table(targets, a, tile_q=, block_k=, num_splits=) -> table (dict); save/load_calib_table (JSON)
  blasst_calibrate_search(gaps, target)                -> (lambda, reached sparsity)
  blasst_calibrate_fit(lambdas, lengths)               -> a
"""
from ._abi import (BlasstError, blasst_abi_version, blasst_calibrate, calib_table,  # noqa: F401
                   load_calib_table, save_calib_table,
                   blasst_calibrate_fit, blasst_calibrate_search, blasst_decode,
                   blasst_decode_gaps, blasst_decode_noalloc, blasst_decode_paged, blasst_decode_paged_plan,
                   blasst_decode_plan, blasst_last_error, blasst_prefill, blasst_prefill_gaps,
                   blasst_status_str, library_path, load_library)

__all__ = [
    "BlasstError", "blasst_prefill", "blasst_prefill_gaps", "blasst_decode", "blasst_decode_gaps", "blasst_decode_plan", "blasst_decode_noalloc",
    "blasst_decode_paged",
    "blasst_decode_paged_plan", "blasst_calibrate",
    "blasst_calibrate_search", "blasst_calibrate_fit", "blasst_status_str", "blasst_last_error",
    "blasst_abi_version", "library_path", "load_library", "calib_table", "save_calib_table", "load_calib_table",
]
