"""MI355X (gfx950) forward pass of the fine-grained gated delta rule (FG2-GDN) and
its KDA, GDN, DeltaProduct and GDN2/RWKV-7-style variants.

The computation lives in libgdn.so (hand-written HIP kernels behind the C ABI of
include/gdn.h); this package is its ctypes binding.
"""
from ._lib import (GdnArgs, GdnError, VARIANTS, gdn_abi_version, gdn_asym_stabilize,  # noqa: F401
                   gdn_chunk_fwd, gdn_chunk_fwd_args, gdn_chunk_fwd_static, gdn_chunk_prepare, gdn_chunk_scan, gdn_final_state,
                   gdn_recurrent_bwd, gdn_recurrent_step, gdn_status_str, gdn_workspace_bytes,
                   load_library,
                   make_args)
