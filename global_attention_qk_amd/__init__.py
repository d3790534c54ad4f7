"""zgattn: hybrid gated sliding-window / global causal GQA attention for MI355X (gfx950).

The compute lives in ``libzgattn.so`` (hand-written HIP kernels behind a C ABI declared
in ``include/zgattn.h``); this package is the thin binding. Importing it does not load the
library; the first call does, and raises if the library has not been built.
"""

from .api import (  # noqa: F401
    global_decode,
    global_decode_noalloc,
    global_decode_workspace_bytes,
    global_prefill,
    global_prefill_varlen,
    global_prefill_varlen_workspace_bytes,
    global_prefill_workspace_bytes,
    make_desc,
    model_decode,
    model_decode_workspace_bytes,
    prefill_backward,
    prefill_backward_workspace_bytes,
    qknorm_rope,
    rotary_dim_for,
    swa_decode,
    swa_prefill,
    swa_prefill_varlen,
)
from ._lib import ZgattnError, lib  # noqa: F401
