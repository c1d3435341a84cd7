"""Pins of the oracle's 4-bit weights (DFlash explainer, section 8: 4 bits in groups of
64; TensorFold #1851, "Exactness", Precision).

Each check is a closed form or a property the affine group quantizer must have, so a
dropped term, a wrong group edge, a wrong rounding or a wrong level count fails one:
planted codes come back exactly, groups are independent, each group's minimum is
exact, the error stays within half a step, and the dequantized product equals the
two-term form scale * sum(x q) + bias * sum(x) the GPU computes.
"""
import numpy as np
import pytest

from oracle import dflash_oracle as O


def test_planted_codes_come_back_exactly():
    # a group b + s * c with s a power of two: the range is exactly 15 s, so the scale
    # is s and every code is recovered, and dequantization is exact
    rng = np.random.default_rng(0)
    N, K = 6, 256
    codes = rng.integers(0, 16, (N, K))
    codes[:, ::64] = 0                       # each group holds its minimum ...
    codes[:, 1::64] = 15                     # ... and its maximum
    s = 2.0 ** rng.integers(-12, -4, (N, K // 64))
    b = -rng.integers(1, 200, (N, K // 64)) * s       # every b + s c is an 8-bit integer times s
    w = b.repeat(64, 1) + s.repeat(64, 1) * codes
    assert np.array_equal(O.round_bf16(w), w)            # bf16 weights
    q, scale, bias = O.quantize_affine(w)
    assert np.array_equal(q, codes) and np.array_equal(scale, s) and np.array_equal(bias, b)
    np.testing.assert_array_equal(O.dequantize_affine(q, scale, bias), w)


def test_groups_are_the_64_weights_of_a_row_and_independent():
    rng = np.random.default_rng(1)
    w = O.round_bf16(rng.normal(0, 0.02, (4, 512)))
    q, s, b = O.quantize_affine(w)
    assert q.shape == w.shape and s.shape == (4, 8) and b.shape == (4, 8)
    assert q.dtype == np.uint8 and q.max() <= 15
    for r in range(4):
        for g in range(8):
            grp = w[r, 64 * g:64 * (g + 1)]
            assert b[r, g] == grp.min()
            assert s[r, g] == O.round_bf16((grp.max() - grp.min()) / 15.0)
    w2 = w.copy()
    w2[2, 130] = 0.5                          # a new maximum in group 2 of row 2 only
    q2, s2, b2 = O.quantize_affine(w2)
    changed = np.argwhere(s2 != s)
    assert changed.tolist() == [[2, 2]]
    mask = np.ones_like(q, dtype=bool)
    mask[2, 128:192] = False
    assert np.array_equal(q2[mask], q[mask])


def test_error_within_half_a_step_and_extremes():
    rng = np.random.default_rng(2)
    w = O.round_bf16(rng.normal(0, 0.02, (64, 1024)) * rng.lognormal(0, 1, (64, 1))).astype(np.float64)
    q, s, b = O.quantize_affine(w)
    d = O.dequantize_affine(q, s, b)
    step = s.repeat(64, 1)
    # rounding to the nearest level: within half a step, plus the few levels past the
    # top that a scale rounded down to bf16 cannot reach (at most 15 * 2^-9 steps)
    assert np.all(np.abs(d - w) <= step * (0.5 + 15 * 2.0 ** -9))
    g = w.reshape(64, 16, 64)
    # every group's smallest weight is code 0 and is represented exactly
    np.testing.assert_array_equal(d.reshape(64, 16, 64).min(-1), g.min(-1))
    assert np.all(q.reshape(64, 16, 64).max(-1) >= 14)


def test_constant_group_has_scale_zero():
    w = np.full((2, 128), 0.25)
    w[1, 64:] = np.linspace(-1, 1, 64)
    w = O.round_bf16(w)
    q, s, b = O.quantize_affine(w)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and s[1, 1] > 0
    assert not q[0].any() and not q[1, :64].any()
    np.testing.assert_array_equal(O.dequantize_affine(q, s, b)[:, :64], w[:, :64])


def test_rounding_is_to_nearest_even_in_float64():
    # codes 1.5 and 2.5 steps above the minimum go to 2 and 2 (ties to even)
    s, lo = 2.0 ** -6, -0.5
    grp = np.full(64, lo)
    grp[1] = lo + 15 * s                      # range exactly 15 steps
    grp[2] = lo + 1.5 * s
    grp[3] = lo + 2.5 * s
    grp[4] = lo + 2.5 * s + 2.0 ** -20        # just above a tie
    q, sc, _ = O.quantize_affine(grp[None])
    assert sc[0, 0] == s
    assert q[0, :5].tolist() == [0, 15, 2, 2, 3]


def test_dequantized_product_is_the_two_term_form():
    # sum_k x_k (bias + scale q_k) over a group = scale * sum x q + bias * sum x: the form
    # the GPU computes (codes through the MFMA, then one scale and one bias per group)
    rng = np.random.default_rng(3)
    x = O.round_bf16(rng.normal(0, 1, (5, 256)))
    w = O.round_bf16(rng.normal(0, 0.02, (7, 256)))
    q, s, b = O.quantize_affine(w)
    direct = x @ O.dequantize_affine(q, s, b).T
    xq = np.einsum("mgk,ngk->mng", x.reshape(5, 4, 64), q.reshape(7, 4, 64).astype(np.float64))
    xs = x.reshape(5, 4, 64).sum(-1)
    two_term = (s[None] * xq + b[None] * xs[:, None, :]).sum(-1)
    np.testing.assert_allclose(direct, two_term, rtol=1e-12, atol=1e-12)


def test_quantized_set_is_every_gemm_weight():
    from types import SimpleNamespace
    cfg = SimpleNamespace(n_layers=2)
    names = O.quantized_names(cfg)
    assert "embed" not in names and "fc" in names and "lm_head" in names
    assert len(names) == 2 + 7 * 2
    assert not any(n.endswith(("norm", "_norm")) for n in names)
