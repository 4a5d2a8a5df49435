"""FlashMap draft-step attention path on MI355X (gfx950).

The compute lives in libfm.so (hand-written HIP kernels behind the C ABI of
include/fm.h); :mod:`.binding` is its ctypes binding, :mod:`.step` runs one
draft step's calls in order, :mod:`.workloads` draws seeded synthetic inputs.
"""

__version__ = "0.1.0"

from .binding import (  # noqa: F401
    FmError,
    KVPool,
    fm_block_self_attention,
    fm_cross_attention_workspace_size,
    fm_last_error,
    fm_paged_cross_attention,
    fm_plan_cross_attention,
    fm_version,
    fm_write_context_kv,
    fm_write_context_kv_workspace_size,
    load_library,
)
