"""CPU oracle for the MARS hot path — test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the product path never does.
"""

from .mars_oracle import (  # noqa: F401
    beta,
    build_mask,
    build_mask_loops,
    causal_mask,
    ar_signal_ratio,
    attn_causal,
    attn_two_stream,
    attn_two_stream_backward,
    attn_block_decode,
    attn_block_decode_rows,
    block_sync_advance,
    block_sync_step,
    block_freeze,
    gather_prefix,
    lmhead,
    confidence,
    confidence_row,
    accept,
    accept_count,
    commit,
    useful_pairs_two_stream,
)
