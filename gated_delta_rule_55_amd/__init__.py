"""KDA (Kimi Delta Attention) forward on AMD MI355X: chunked prefill and
recurrent decode as hand-written HIP kernels behind a C ABI (include/kda.h)."""
from .kda import (  # noqa: F401
    chunk_prefill,
    prefill_workspace_bytes,
    recurrent_decode,
    recurrent_prefill,
    workspace_status,
)
from ._abi import KdaError, LIB_PATH  # noqa: F401
