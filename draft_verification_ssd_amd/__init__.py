"""MI355X (gfx950) library for batched lossless draft verification and the SSD / Saguaro pieces.

The compute lives in libssd.so (hand-written HIP, C ABI in include/ssd.h); this package is the thin
ctypes binding over it plus the build step. See ``_lib`` for the entry points.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    FLAG_BAD_C,
    FLAG_BAD_F,
    FLAG_BAD_TOKEN,
    FLAG_SAGUARO_NORM,
    LIB_PATH,
    SSD_BF16,
    SSD_ERR_HIP,
    SSD_ERR_INVALID_ARG,
    SSD_ERR_UNSUPPORTED,
    SSD_ERR_WORKSPACE,
    SSD_F32,
    SSD_OK,
    VerifyCall,
    Workspace,
    lib,
    ssd_cache_keys,
    ssd_cache_lookup,
    ssd_fanout_alloc,
    ssd_read_flags,
    ssd_saguaro_adjust,
    ssd_saguaro_sample,
    ssd_saguaro_sample_workspace_bytes,
    ssd_saguaro_topf,
    ssd_saguaro_topf_workspace_bytes,
    ssd_saguaro_workspace_bytes,
    ssd_topf_guess,
    ssd_topf_workspace_bytes,
    ssd_verify,
    ssd_verify_launches,
    ssd_verify_workspace_bytes,
)
