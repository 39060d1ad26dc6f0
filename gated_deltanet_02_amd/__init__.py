"""MI355X-native chunked Gated DeltaNet prefill.

The compute lives in ``libgdn.so`` (gfx950 HIP kernels behind the C ABI in
``include/gdn.h``); this package only marshals torch tensors into that ABI.
Importing the package does not load the library; the first call does, and
raises if it was not built.
"""
from ._binding import (GdnError, GdnOptions, GdnTensor, GdnWorkspaceLayout,  # noqa: F401
                       STAGE_ALL, STAGE_SCAN, STAGE_TABLE, STAGE_WY, EXPORTED,
                       SCAN_AUTO, SCAN_ONE_PASS, SCAN_TWO_LEVEL, FLAG_BETA_LOGITS,
                       FLAG_DECAY_PROJ, FLAG_OUTPUT_GATE, FLAG_QKV_SILU, FLAG_QKV_CONV, gdn_output_gate,
                       gdn_check_cu_seqlens,
                       alloc_workspace, describe, gdn_abi_version,
                       gdn_default_options, gdn_get_workspace_layout,
                       gdn_decode, gdn_last_error, gdn_prefill, gdn_prefill_ex,
                       gdn_prefill_noalloc, NOALLOC_SCRATCH_BYTES,
                       gdn_status_string, gdn_workspace_size, library_path,
                       options)
from ._binding import GraphCache, PreparedPrefill  # noqa: F401,E402
