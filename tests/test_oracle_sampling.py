"""Pins of the oracle's sampling functions (DFlash explainer, section 4, "Sampling
decoding") against what the mathematics fixes.

None of these re-types the oracle's formulas: the inverse-CDF draw is checked on
weights whose bins are known exactly; the acceptance rule by the property the page
states for it (the emitted token follows the target's distribution, "lossless"),
integrated over a grid of uniforms; and the greedy rule as its zero-temperature limit
(the greedy oracle has its own pins).
"""
import numpy as np
import pytest

from oracle import dflash_oracle as O


def test_inverse_cdf_bins_on_exact_weights():
    # weights 1, 2, 3, 4 (sum 10): id k owns u in [c_{k-1}, c_k) / 10
    w = np.array([1.0, 2.0, 3.0, 4.0])
    for u, k in [(0.0, 0), (0.05, 0), (0.0999, 0), (0.1001, 1), (0.2999, 1), (0.3001, 2), (0.5999, 2),
                 (0.6001, 3), (0.9999, 3)]:
        assert O.sample_index(w, u) == k, (u, k)
    # scale does not matter
    assert all(O.sample_index(7.0 * w, u) == O.sample_index(w, u) for u in np.linspace(0, 0.999, 97))


def test_inverse_cdf_never_draws_a_zero_weight():
    w = np.array([0.0, 0.5, 0.0, 0.0, 0.5, 0.0])
    got = {O.sample_index(w, u) for u in np.linspace(0.0, 0.9999, 1001)}
    assert got == {1, 4}
    assert O.sample_index(w, 0.0) == 1


def test_inverse_cdf_frequencies_over_a_uniform_grid():
    rng = np.random.default_rng(3)
    w = rng.random(7)
    n = 20000
    u = (np.arange(n) + 0.5) / n
    counts = np.bincount([O.sample_index(w, x) for x in u], minlength=7)
    assert np.max(np.abs(counts / n - w / w.sum())) <= 2.0 / n


def test_tempered_probs_limits():
    x = np.array([1.0, 3.0, 2.0, 3.0])
    # T -> infinity: uniform; T = 1: the plain softmax; T -> 0: the argmax set, evenly
    assert np.allclose(O.tempered_probs(x, 1e9), 0.25)
    assert np.allclose(O.tempered_probs(x, 1.0), np.exp(x) / np.exp(x).sum())
    assert np.allclose(O.tempered_probs(x, 1e-3), [0.0, 0.5, 0.0, 0.5])


def _one_position(dl, tl_row0, tl_row1, d, T, ua, us):
    """verify_sampling on one stream with a single drafted token (B = 2)."""
    acc, tok, com = O.verify_sampling(np.array([[d]]), dl[None, None, :], np.stack([tl_row0, tl_row1])[None],
                                      T, np.array([[ua]]), np.array([us]))
    return int(acc[0]), int(tok[0]), com[0]


@pytest.mark.parametrize("seed,T", [(0, 1.0), (1, 0.7), (2, 1.6)])
def test_first_emitted_token_follows_the_target_distribution(seed, T):
    # The page's losslessness: whatever the draft, the first token the round emits
    # (d_1 if accepted, else the residual draw) is distributed as the target's q_0.
    # Integrate exactly over the draft draw and numerically over a midpoint grid of
    # the acceptance and residual uniforms.
    rng = np.random.default_rng(seed)
    V = 5
    dl, t0, t1 = rng.normal(0, 1.5, V), rng.normal(0, 1.5, V), rng.normal(0, 1.5, V)
    p = np.exp(dl / T) / np.exp(dl / T).sum()
    q = np.exp(t0 / T) / np.exp(t0 / T).sum()
    n = 400
    grid = (np.arange(n) + 0.5) / n
    emitted = np.zeros(V)
    for d in range(V):
        acc_rate = np.mean([_one_position(dl, t0, t1, d, T, ua, 0.5)[0] for ua in grid])
        rejected_draws = np.bincount([_one_position(dl, t0, t1, d, T, 1.0 - 1e-12, us)[1] for us in grid],
                                     minlength=V) / n
        emitted[d] += p[d] * acc_rate
        emitted += p[d] * (1.0 - acc_rate) * rejected_draws
    assert np.max(np.abs(emitted - q)) < 4.0 / n, (emitted, q)


def test_accepting_everything_when_draft_and_target_agree():
    rng = np.random.default_rng(5)
    S, B, V, T = 3, 5, 11, 0.9
    logits = rng.normal(0, 1, (S, B, V))
    draft_logits = logits[:, :B - 1]
    draft = rng.integers(0, V, (S, B - 1))
    ua = rng.random((S, B - 1))
    us = rng.random(S)
    acc, tok, com = O.verify_sampling(draft, draft_logits, logits, T, ua, us)
    assert np.all(acc == B - 1)
    for s in range(S):
        w = np.exp(logits[s, B - 1] / T)
        c = np.cumsum(w / w.sum())
        assert c[tok[s] - 1] <= us[s] < c[tok[s]] if tok[s] > 0 else us[s] < c[0]
        assert list(com[s]) == list(draft[s]) + [tok[s]]


def test_zero_temperature_limit_is_greedy_verify():
    rng = np.random.default_rng(9)
    S, B, V = 4, 6, 40
    # well-separated logits: the tempered distributions are one-hot at the argmax
    dl = rng.permutation(np.arange(S * (B - 1) * V)).reshape(S, B - 1, V).astype(np.float64)
    tl = rng.permutation(np.arange(S * B * V)).reshape(S, B, V).astype(np.float64)
    draft = np.argmax(dl, -1)
    target = np.argmax(tl, -1)
    # make some leading drafts agree with the target
    for s in range(S):
        k = s % (B - 1)
        draft[s, :k] = target[s, :k]
        for j in range(k):
            dl[s, j, target[s, j]] = dl[s, j].max() + 1.0
    acc, tok, com = O.verify_sampling(draft, dl, tl, 1e-3, rng.random((S, B - 1)), rng.random(S))
    ga, gb, gc = O.verify_greedy(draft, target)
    assert np.array_equal(acc, ga) and np.array_equal(tok, gb) and np.array_equal(com, gc)


def test_rejected_draft_token_is_never_redrawn_when_the_target_excludes_it():
    V, T = 6, 1.0
    dl = np.zeros(V)
    t0 = np.zeros(V)
    t0[2] = -np.inf            # the target gives id 2 no mass
    for us in np.linspace(0, 0.999, 50):
        a, tok, com = _one_position(dl, t0, np.zeros(V), 2, T, 0.3, us)
        assert a == 0 and tok != 2 and com[0] == tok and com[1] == -1
