"""The float64 model's own sensitivity to bf16 rounding: how far the oracle's logits move
when a seeded fraction of its stored (rounded) elements is rounded the other way.

Test infrastructure shared by the CPU conditioning pins and the GPU whole-round tests.
It wraps the oracle's storage rounding; the oracle itself is not modified.
"""
import numpy as np

from oracle import dflash_oracle as O


def ulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 7), 2.0 ** -133)


def with_flips(fn, rate, seed):
    """Run fn() with every bf16 storage rounding of the oracle moved by one ulp (toward
    the unrounded value's side) at a seeded fraction `rate` of the elements."""
    orig = O.round_to
    rng = np.random.default_rng(seed)

    def flippy(x, dtype):
        y = orig(x, dtype)
        if dtype != "bf16":
            return y
        m = rng.random(np.shape(y)) < rate
        return np.where(m, y + np.where(np.asarray(x) >= y, 1.0, -1.0) * ulp_bf16(y), y)

    O.round_to = flippy
    try:
        return fn()
    finally:
        O.round_to = orig


def movement(base_logits, flipped_logits):
    """(max, mean) absolute logit movement over paired lists of [rows, V] arrays."""
    mx = max(float(np.max(np.abs(a - b))) for a, b in zip(base_logits, flipped_logits))
    mn = max(float(np.mean(np.abs(a - b))) for a, b in zip(base_logits, flipped_logits))
    return mx, mn


# The whole-round bar of the wide presets: tol = max(2e-2, FACTOR x the oracle's own max
# logit movement at RATE); both constants are pinned by tests/test_oracle_conditioning.py.
RATE = 1e-4
FACTOR = 2.0
