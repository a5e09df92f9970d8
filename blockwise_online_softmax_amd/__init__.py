"""MI355X (gfx950) ring attention: blockwise online softmax behind a C ABI.

The computation lives in libra.so (HIP kernels for gfx950, C ABI in
include/ra.h).  This package is the thin Python binding: `capi` mirrors the
C calls (ra_state_init, ra_block_step, ra_finalize, ra_ring, ra_permute,
ra_positions, ra_state_merge, ra_merge, the vocab-parallel cross-entropy
calls ra_vocab_ce*, and ra_xcd_plan / ra_xcd_speeds for the work split over
the GPU's XCDs) and marshals PyTorch tensors, which serve only as device
memory and streams.  Build the library with
`python -m blockwise_online_softmax_amd.build`.
"""

from .capi import (  # noqa: F401
    RA_BF16, RA_F32, RA_MASK_CAUSAL, RA_MASK_NONE, RA_CONTIGUOUS, RA_STRIPED, RA_ZIGZAG,
    LAYOUT_IDS, State, load, last_error, ra_block_step, ra_finalize, ra_layout_position, ra_merge,
    ra_permute,
    ra_positions, ra_ring, ra_ring_workspace_bytes, ra_state_init, ra_state_merge, ra_version,
    ra_vocab_ce, ra_vocab_ce_combine, ra_vocab_ce_grad, ra_vocab_ce_shard, ra_vocab_ce_static,
    ra_vocab_ce_workspace_bytes, ra_xcd_plan, ra_xcd_speeds,
    ring_attention,
)
