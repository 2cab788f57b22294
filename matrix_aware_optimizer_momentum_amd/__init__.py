"""MI355X-native Muon-family optimizer step (Sign-Muon, CacheMuon, LionMuon).

The step runs in the HIP library libsm.so (C ABI in include/sm.h); this
package is its Python binding.  Importing it does not load the library; the
first call does, and fails loudly if it has not been built.
"""
from ._binding import (BF16, CACHE_MUON, ENC_BITS, ENC_INT8, F32, LION_MUON, MODE_FORCE_FRESH,
                       MODE_FORCE_REUSE, MODE_TRIGGER, SIGN_MUON, UPDATE_POLAR, UPDATE_VOTE,
                       SmError, lib)
from .api import (MatrixBuffers, NSParams, StepCall, StepConfig, StepGraph, gram_ns_cached,
                  gram_ns_cached_ws, mfma_ceiling, ns_polar, ns_polar_noalloc, ns_polar_ws, polar_update, profile_enable,
                  profile_read, profile_read_bytes, profile_reset, sign_int8, sign_pack, spectral_norm, step, step_ws,
                  vote, vote_update, vote_update_int8)

__all__ = [
    "BF16", "CACHE_MUON", "ENC_BITS", "ENC_INT8", "F32", "LION_MUON", "MODE_FORCE_FRESH",
    "MODE_FORCE_REUSE", "MODE_TRIGGER", "SIGN_MUON", "UPDATE_POLAR", "UPDATE_VOTE", "SmError",
    "lib", "MatrixBuffers", "NSParams", "StepCall", "StepConfig", "StepGraph", "gram_ns_cached",
    "gram_ns_cached_ws", "mfma_ceiling", "ns_polar", "ns_polar_noalloc", "ns_polar_ws", "polar_update", "profile_enable",
    "profile_read", "profile_read_bytes", "profile_reset", "sign_int8", "sign_pack", "spectral_norm", "step",
    "step_ws", "vote",
    "vote_update", "vote_update_int8",
]
