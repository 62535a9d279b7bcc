"""Seeded synthetic inputs for the KDA verify/commit path (no method arithmetic)."""

from .configs import (  # noqa: F401
    Batch,
    DeferredRun,
    CONFIG_NAMES,
    SINGLE_CALL,
    make_batch,
    make_deferred,
    bf16_from_f32,
    bf16_to_f32,
)
