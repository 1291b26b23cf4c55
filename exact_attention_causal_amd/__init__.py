"""Exact causal attention (FlashAttention-2 forward and backward) for MI355X.

The computation lives in hand-written HIP kernels for gfx950 behind the C ABI
in ``include/fa.h`` (``libfa_mi355x.so``); :mod:`.fa` is its ctypes binding.
"""
from .fa import (FA_BF16, FA_F32, HEAD_DIMS, FaError, FlashAttention, Plan, backward,
                 backward_partial, fa_bwd, fa_bwd_noalloc, fa_bwd_partial, fa_bwd_preprocess,
                 fa_bwd_workspace_size, fa_fwd, fa_fwd_partial, fa_fwd_workspace_size, fa_fwd_ws,
                 fa_get_plan, fa_merge, fa_strerror, flash_attention, forward, forward_partial,
                 forward_split_kv, load_library, merge, split_chunk)

__all__ = ["FA_BF16", "FA_F32", "HEAD_DIMS", "FaError", "FlashAttention", "Plan", "backward",
           "backward_partial", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_partial", "fa_bwd_preprocess",
           "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_partial", "fa_fwd_workspace_size", "fa_fwd_ws",
           "fa_get_plan", "fa_merge", "fa_strerror", "flash_attention", "forward", "forward_partial",
           "forward_split_kv", "load_library", "merge", "split_chunk"]
