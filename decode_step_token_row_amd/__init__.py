"""decode_step_token_row_amd -- on-device batched token sampling for MI355X.

The work runs in libarcs.so (hand-written HIP for gfx950, C ABI in
include/arcs.h); this package is the thin Python binding over it.
"""

from ._binding import (  # noqa: F401
    ArcsError,
    DTYPE_BF16,
    DTYPE_F32,
    LIB_PATH,
    ROW_PARAMS_DTYPE,
    ROW_STATS_DTYPE,
    argmax,
    commit_tokens,
    library,
    make_key,
    params_to_device,
    sample,
    sample_debug,
    sample_keyed,
    status_string,
    top_logprobs,
    version,
    workspace_bytes,
)
from ._binding import (  # noqa: F401
    PATH_CUTOFF,
    PATH_GREEDY,
    PATH_MINP_FLOOR,
    PATH_PENALTY,
    PATH_RESIDENT,
    PATH_REREAD,
    PATH_SORT_SKIP,
    PATH_SPECIAL,
    PATH_TIE_SPLIT,
    ROW_BAD_FLAGS,
    ROW_BAD_MIN_P,
    ROW_BAD_PENALTY,
    ROW_BAD_TEMPERATURE,
    ROW_BAD_TOP_P,
    ROW_HISTORY_TOO_LONG,
    ROW_OK,
    ROW_VOCAB_TOO_LARGE,
    MAX_HISTORY,
    MAX_PENALTY_VOCAB,
)
