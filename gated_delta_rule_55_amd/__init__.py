"""KDA (Kimi Delta Attention) forward on AMD MI355X: chunked prefill and
recurrent decode, and the short causal conv before them, as hand-written HIP
kernels behind a C ABI (include/kda.h, include/kda_conv.h)."""
from .kda import (  # noqa: F401
    causal_conv1d_fwd,
    causal_conv1d_update,
    chunk_prefill,
    prefill_workspace_bytes,
    recurrent_decode,
    recurrent_prefill,
    workspace_status,
)
from ._abi import KdaError, LIB_PATH  # noqa: F401
