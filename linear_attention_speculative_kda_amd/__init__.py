"""KDA speculative verify + accepted-token commit ("RecoverSSM") on MI355X.

The computation lives in libkda.so (hand-written HIP for gfx950, C ABI in
include/kda.h); this package is its Python front end. Importing it does not
touch the GPU; the first call loads the library and fails loudly if it has
not been built.
"""

from .kda import (  # noqa: F401
    HEAD_DIM,
    Align,
    Layer,
    Records,
    allocate_records,
    MAX_LAYERS,
    check_rows,
    kda_commit,
    kda_commit_layers,
    kda_conv_compact,
    kda_flush,
    kda_flush_layers,
    kda_recurrent,
    kda_recurrent_spec,
    kda_verify,
    kda_verify_deferred,
)
from ._lib import KdaError, LIB_PATH, load  # noqa: F401
