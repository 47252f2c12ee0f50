"""MI355X (gfx950) fused attention forward with the online-softmax recurrence.

The computation lives in libfa.so (hand-written HIP kernels behind the C ABI of
include/fa.h); this package only marshals torch tensors into that ABI.
"""
from .fa import (EXPORTS, FA_BF16, FA_ERR_HIP, FA_ERR_INVALID_ARG, FA_ERR_SCRATCH_LIMIT,
                 FA_ERR_UNSUPPORTED, FA_F32, fa_decode_scratch_bytes, fa_decode_splitkv_noalloc,
                 FA_OK, FaError, attention, attention_backward, attention_v1, bind_backward,
                 bind_forward, decode, fa_backward,
                 fa_forward_v1, fa_forward_v1_workspace_bytes,
                 fa_backward_workspace_bytes, fa_decode_splitkv, fa_decode_workspace_bytes,
                 fa_forward, fa_softmax, fa_softmax_workspace_bytes, load_library, softmax,
                 status_str, testing_set_softmax_spin_limit, testing_set_rescale_rule,
                 RESCALE_EAGER, RESCALE_THRESHOLD, RESCALE_GUARD, probe_mfma, probe_read, probe_copy,
                 PROBE_MFMA_FLOPS, PROBE_THREADS)

__all__ = ["EXPORTS", "FA_BF16", "FA_ERR_HIP", "FA_ERR_INVALID_ARG", "FA_ERR_SCRATCH_LIMIT",
           "FA_ERR_UNSUPPORTED", "FA_F32", "fa_decode_scratch_bytes", "fa_decode_splitkv_noalloc",
           "FA_OK", "FaError", "attention", "attention_backward", "attention_v1", "bind_backward",
           "bind_forward", "decode",
           "fa_backward", "fa_forward_v1", "fa_forward_v1_workspace_bytes",
           "fa_backward_workspace_bytes", "fa_decode_splitkv",
           "fa_decode_workspace_bytes", "fa_forward", "fa_softmax", "fa_softmax_workspace_bytes",
           "load_library", "softmax", "status_str", "testing_set_softmax_spin_limit",
           "testing_set_rescale_rule", "RESCALE_EAGER", "RESCALE_THRESHOLD", "RESCALE_GUARD",
           "probe_mfma", "probe_read", "probe_copy", "PROBE_MFMA_FLOPS", "PROBE_THREADS"]
