"""MI355X-native TTT-layer library (HIP kernels for gfx950 behind a C ABI).

The entry points mirror include/ttt.h:
  * forward: ttt_forward_fullbatch, ttt_forward_fullbatch_epochs (several full-batch epochs),
    ttt_forward_chunked_causal, ttt_forward_chunked_bidir, ttt_forward_chunked_bidir2d (raster-
    and column-order bidirectional scans), ttt_mlp_forward;
  * backward (the layers' gradients for the outer loop): ttt_backward_fullbatch,
    ttt_backward_chunked_causal, ttt_backward_chunked_bidir;
  * around the layer: ttt_dwconv3x3 (the depth-wise 3x3 convolution over the token grid that
    precedes a scan or runs beside it), ttt_block_epilogue (ViT^3's gated branch and convolution
    branch concatenated and projected);
  * ttt_forward_fullbatch_noalloc (full-batch with the library's static scratch instead of a
    workspace, for callers that cannot allocate) and ttt_workspace_size.
"""
from .ttt import (  # noqa: F401
    TTT_BF16, TTT_F32, TTT_NOALLOC_SCRATCH_BYTES, TTT_OP_BIDIR, TTT_OP_CAUSAL, TTT_OP_FULLBATCH,
    TTT_OP_BIDIR2D, TTT_OP_BIDIR_BWD, TTT_OP_CAUSAL_BWD, TTT_OP_FULLBATCH_BWD, TTT_OP_MLP,
    TTTError, load_library, status_string, ttt_backward_chunked_bidir, ttt_backward_chunked_causal,
    ttt_backward_fullbatch, ttt_block_epilogue, ttt_forward_chunked_bidir, ttt_forward_chunked_bidir2d, ttt_forward_chunked_causal,
    ttt_dwconv3x3, ttt_forward_fullbatch, ttt_forward_fullbatch_epochs, ttt_forward_fullbatch_noalloc, ttt_mlp_forward, ttt_workspace_size)
