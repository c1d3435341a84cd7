"""Pins of the oracle's DFlash2 candidate path selector (DFlash explainer, section 5;
TensorFold #1851 item 1; Strata #3457, "Problem and result": --spec-min-p).

Checked against what fixes it: with rank 0 (no codebooks) the edge term is zero and
the path is each position's own top-1 (TensorFold #1851 item 1), the best path equals
an exhaustive search over every candidate path, candidates are the top-k in logit
order with ties to the lowest id, a planted pair score moves the path, and the min-p
stop cuts the draft exactly where the chosen token's probability first falls below it.
"""
import itertools

import numpy as np

from oracle import dflash_oracle as O


def test_rank_zero_is_each_positions_top1():
    rng = np.random.default_rng(0)
    logits = rng.normal(0, 1.3, (15, 3000))
    toks, n = O.select_path(logits, None, None, 16, 0.0)
    assert n == 15 and np.array_equal(toks, O.argmax_lowest(logits))
    empty = np.zeros((3000, 0))
    assert np.array_equal(O.select_path(logits, empty, empty, 16, 0.0)[0], toks)


def test_best_path_by_exhaustive_search():
    rng = np.random.default_rng(1)
    V, r, k = 40, 6, 3
    for trial in range(20):
        logits = rng.normal(0, 1.0, (4, V))
        U, W = rng.normal(0, 0.8, (V, r)), rng.normal(0, 0.8, (V, r))
        toks, n = O.select_path(logits, U, W, k, 0.0)
        cand = [np.argsort(-l, kind="stable")[:k] for l in logits]
        lsm = [l - np.log(np.sum(np.exp(l - l.max()))) - l.max() for l in logits]
        best, arg = -np.inf, None
        for path in itertools.product(range(k), repeat=4):
            c = [cand[j][path[j]] for j in range(4)]
            sc = sum(lsm[j][c[j]] for j in range(4)) + sum(U[c[j]] @ W[c[j + 1]] for j in range(3))
            if sc > best:
                best, arg = sc, c
        assert n == 4 and list(toks) == arg, trial


def test_candidates_in_logit_order_ties_to_lowest_id():
    l = np.array([0.5, 2.0, 2.0, 1.0, 2.0, -1.0])
    assert list(O.top_k_ordered(l, 4)) == [1, 2, 4, 3]


def test_a_planted_pair_score_moves_the_path():
    V = 10
    logits = np.full((3, V), -5.0)
    logits[:, 0], logits[:, 1] = 1.0, 0.9         # every position: 0 first, 1 second ...
    logits[2, 1] = 0.5                             # ... the last one more firmly
    U, W = np.zeros((V, 1)), np.zeros((V, 1))
    assert list(O.select_path(logits, U, W, 2, 0.0)[0]) == [0, 0, 0]
    U[0, 0], W[1, 0] = 1.0, 1.0                    # the pair (0 then 1) scores +1
    # one 0 -> 1 step is worth it; taking it at the last position would cost 0.5, not 0.1
    assert list(O.select_path(logits, U, W, 2, 0.0)[0]) == [0, 1, 0]


def test_min_p_stop():
    logits = np.log(np.array([[0.9, 0.1], [0.6, 0.4], [0.3, 0.7], [0.55, 0.45]]))
    toks, n = O.select_path(logits, None, None, 2, 0.0)
    assert n == 4 and list(toks) == [0, 0, 1, 0]
    toks, n = O.select_path(logits, None, None, 2, 0.58)       # p = 0.9, 0.6, 0.7, 0.55
    assert n == 3 and list(toks) == [0, 0, 1, -1]
    toks, n = O.select_path(logits, None, None, 2, 0.65)
    assert n == 1 and list(toks) == [0, -1, -1, -1]
    toks, n = O.select_path(logits, None, None, 2, 1.5)
    assert n == 0 and list(toks) == [-1] * 4
    # a stopped draft verifies no further than its length
    acc, _, _ = O.verify_greedy(np.array([[0, 0, 1, -1]]), np.array([[0, 0, 1, 0, 5]]))
    assert acc[0] == 3
