"""Seeded synthetic workloads for the DFlash draft round.

This package holds only shapes and seeded random inputs. It contains none of
the round's arithmetic, so both the CPU oracle and the HIP path can take their
inputs from it without sharing any computation.
"""
from .presets import PRESETS, Preset, preset  # noqa: F401
from .synth import (  # noqa: F401
    make_weights, make_taps, make_context_taps, make_context_kv, make_page_table, make_anchor,
    make_target_rows, draw_accept_lengths, round_rows, tensor_names, ctx_lens,
    tensor_shape, LAYER_TENSORS,
)
