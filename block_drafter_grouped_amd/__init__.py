"""MI355X (gfx950) draft-block hot path of DFlash2 speculative decoding.

The compute lives in ``libdflash2.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/dflash2.h``).  ``dflash2`` is a thin ctypes
binding with the same entry points; it only marshals arguments.  PyTorch is
used by callers for device memory and streams.
"""
from .dflash2 import (  # noqa: F401
    DFS_BF16,
    DFS_F32,
    Config,
    DFSError,
    STATUS,
    STATIC_WORKSPACE_BYTES,
    SelectOpts,
    WALKS,
    conv,
    conv_layers,
    conv_layers_workspace_size,
    draft_block,
    draft_block_static,
    head_topk,
    lib,
    select,
    topk_logits,
    validate_config,
    workspace_size,
)
