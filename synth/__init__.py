"""Seeded synthetic inputs for the FastGen profiling / compaction / decode path.

This package only *draws* inputs (Q, K, V, token classes, decode streams).  It
holds none of the method's arithmetic: no softmax, no cumulative scores, no
budgets, no policy levels.  Both the HIP path and the CPU oracle consume what
it produces, and it is the only code they share.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    TOKEN_NORMAL,
    TOKEN_PUNCT,
    TOKEN_SPECIAL,
    ConfigSpec,
    DecodeStream,
    LayerInputs,
    bf16_bits,
    head_types,
    make_decode_stream,
    make_layer,
    round_to_bf16,
    token_classes,
)
