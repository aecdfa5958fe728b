"""MI355X-native TTT-layer forward library (HIP kernels for gfx950 behind a C ABI).

The entry points mirror include/ttt.h: ttt_forward_fullbatch, ttt_forward_chunked_causal,
ttt_forward_chunked_bidir, ttt_mlp_forward, ttt_workspace_size.
"""
from .ttt import (  # noqa: F401
    TTT_BF16, TTT_F32, TTT_OP_BIDIR, TTT_OP_CAUSAL, TTT_OP_FULLBATCH, TTT_OP_MLP, TTTError, load_library,
    status_string, ttt_forward_chunked_bidir, ttt_forward_chunked_causal, ttt_forward_fullbatch, ttt_mlp_forward,
    ttt_workspace_size)
