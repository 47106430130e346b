"""MARS hot path on MI355X (gfx950): two-stream masked attention (forward and
backward), block-decode attention, LM-head confidence and left-to-right
acceptance with KV commit.

The compute lives in libmars.so (hand-written HIP kernels behind a C ABI, see
include/mars.h); this package is a thin ctypes binding with the same names.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    MARS_BF16,
    MARS_F32,
    MarsError,
    STATUS_BAD_PAGE,
    STATUS_CACHE_OVERFLOW,
    STATUS_NONFINITE,
    lib,
    strerror,
)
from .api import (  # noqa: F401
    mars_accept_commit,
    mars_accept_commit_layers,
    mars_attn_block_decode,
    mars_attn_causal,
    mars_attn_two_stream,
    mars_attn_two_stream_bwd,
    mars_decode_workspace_bytes,
    mars_kv_append,
    mars_block_sync_accept,
    mars_block_freeze,
    mars_lmhead_confidence,
    mars_lmhead_confidence_noalloc,
    mars_lmhead_pack,
    PackedLMHead,
    mars_lmhead_workspace_bytes,
)

__version__ = "0.1.0"
