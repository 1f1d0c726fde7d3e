"""MI355X-native chunked gated delta-rule forward and backward passes (KDA and GDN).

The computation lives in libkda.so (HIP kernels for gfx950 behind the C ABI
of include/kda.h); this package is its thin Python binding.  Build the
library with ``python -m chunked_gated_delta_kda_amd.build``.
"""
from ._binding import (EXPORTS, LIB_PATH, LibKdaError, bwd_workspace_size, gdn_bwd,
                       gdn_bwd_saved, gdn_decode, gdn_fwd, gdn_fwd_save, gdn_fwd_split, gdn_prep, kda_bwd,
                       kda_bwd_saved, kda_decode, kda_fwd, kda_fwd_noalloc, kda_fwd_save, kda_fwd_split,
                       kda_prep,
                       kda_recur, load,
                       status_str, version, workspace_size)
from .autograd import chunk_gdn, chunk_kda

__all__ = ["chunk_kda", "chunk_gdn", "kda_fwd", "gdn_fwd", "kda_fwd_split", "gdn_fwd_split",
           "kda_fwd_noalloc",
           "kda_prep", "gdn_prep", "kda_recur",
           "kda_decode", "gdn_decode", "kda_fwd_save", "gdn_fwd_save", "kda_bwd_saved",
           "gdn_bwd_saved", "kda_bwd", "gdn_bwd", "workspace_size", "bwd_workspace_size",
           "status_str", "version", "load", "LibKdaError", "EXPORTS", "LIB_PATH"]
