"""MI355X-native chunked gated delta-rule forward pass (KDA and GDN).

The computation lives in libkda.so (HIP kernels for gfx950 behind the C ABI
of include/kda.h); this package is its thin Python binding.  Build the
library with ``python -m chunked_gated_delta_kda_amd.build``.
"""
from ._binding import (EXPORTS, LIB_PATH, LibKdaError, gdn_decode, gdn_fwd, gdn_prep, kda_decode,
                       kda_fwd, kda_prep, kda_recur, load, status_str, version, workspace_size)

__all__ = ["kda_fwd", "gdn_fwd", "kda_prep", "gdn_prep", "kda_recur", "kda_decode", "gdn_decode",
           "workspace_size", "status_str", "version", "load", "LibKdaError", "EXPORTS", "LIB_PATH"]
