"""Pins for the oracle's generator, top-k, log-normaliser and draws (CPU only).

Top-k per position follows "DFlash vs DFlash 2", "The candidate selector"; the
draft draw follows "The problem: one expensive token at a time" (the drafter
proposes y from q).  Pins: numpy's Philox (library), numpy lexsort/argmax
(library), scipy logsumexp/softmax (library), numpy searchsorted for the
inverse CDF (library), closed forms and a chi-square frequency check.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax
from scipy.stats import chi2

import oracle

MASK64 = (1 << 64) - 1


def _ctr_minus_one(c):
    v = sum(int(w) << (64 * i) for i, w in enumerate(c)) - 1
    v &= (1 << 256) - 1
    return np.array([(v >> (64 * i)) & MASK64 for i in range(4)], dtype=np.uint64)


@pytest.mark.parametrize("ctr,key", [
    ([1, 0, 0, 0], [0, 0]),
    ([0, 0, 0, 0], [0, 0]),            # borrow through all four words in numpy's form
    ([0, 5, 0, 0], [7, 9]),            # borrow into word 1
    ([123456789, 2, 3, 4], [2 ** 63 + 5, 2 ** 64 - 1]),
    ([2 ** 64 - 1, 2 ** 64 - 1, 17, 1], [42, 0]),
])
def test_philox_matches_numpy(ctr, key):
    """numpy.random.Philox pre-increments its 256-bit counter, so a generator
    created with counter c-1 returns the block of counter c first."""
    bg = np.random.Philox(counter=_ctr_minus_one(ctr), key=np.array(key, dtype=np.uint64))
    ref = bg.random_raw(4)
    got = oracle.philox4x64_10(ctr, key)
    np.testing.assert_array_equal(got, ref.astype(np.uint64))


def test_uniform_layout_and_range():
    for seed, step, b, row, purpose in [(0, 0, 0, 0, 0), (5, 3, 31, 7, 2), (2 ** 40, 99, 1, 15, 1)]:
        bg = np.random.Philox(counter=_ctr_minus_one([step, b, row, purpose]), key=np.array([seed, 0], dtype=np.uint64))
        w0 = int(bg.random_raw(4)[0])
        u = oracle.uniform(seed, step, b, row, purpose)
        assert u == (w0 >> 11) * 2.0 ** -53
        assert 0.0 <= u < 1.0


def test_uniforms_are_uniform():
    us = np.array([oracle.uniform(3, s, 1, 2, 1) for s in range(20000)])
    hist, _ = np.histogram(us, bins=20, range=(0, 1))
    stat = ((hist - 1000.0) ** 2 / 1000.0).sum()
    assert stat < chi2.ppf(1 - 1e-6, 19)


def test_topk_matches_lexsort_with_ties():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((6, 500)).round(1)  # many exact ties
    idx, val = oracle.topk(z, 16)
    for r in range(6):
        order = np.lexsort((np.arange(500), -z[r]))[:16]
        np.testing.assert_array_equal(idx[r], order)
        np.testing.assert_array_equal(val[r], z[r, order])


def test_topk_one_is_first_argmax():
    z = np.array([[1.0, 3.0, 3.0, -2.0], [5.0, 5.0, 5.0, 5.0]])
    idx, _ = oracle.topk(z, 1)
    assert idx[:, 0].tolist() == [int(np.argmax(z[0])), int(np.argmax(z[1]))] == [1, 0]
    assert oracle.argmax(z[0]) == 1 and oracle.argmax(z[1]) == 0


def test_topk_all_equal_row_is_index_order():
    idx, _ = oracle.topk(np.zeros((1, 50)), 10)
    assert idx[0].tolist() == list(range(10))


@pytest.mark.parametrize("T", [1.0, 0.7, 0.05, 3.0])
def test_logsumexp_matches_scipy(T):
    z = np.random.default_rng(1).normal(0, 3, 151936)
    assert abs(oracle.logsumexp(z, T) - logsumexp(z / T)) < 1e-10


def test_logsumexp_constant_row_closed_form():
    z = np.full(1000, 2.5)
    assert abs(oracle.logsumexp(z, 0.5) - (5.0 + np.log(1000))) < 1e-12


def test_categorical_integer_weights_exact_cells():
    w = np.array([0.0, 3.0, 0.0, 1.0, 4.0, 0.0, 2.0])
    c = np.cumsum(w)
    S = c[-1]
    for i in np.nonzero(w)[0]:
        lo = c[i] - w[i]
        for frac in (0.0, 0.25, 0.999):
            u = (lo + frac * w[i]) / S
            assert oracle.categorical(w, u) == i
    assert oracle.categorical(w, 0.0) == 1  # first positive weight


def test_categorical_matches_searchsorted():
    rng = np.random.default_rng(2)
    w = rng.exponential(size=1000) * (rng.random(1000) < 0.7)
    c = np.cumsum(w)
    for u in rng.random(2000):
        ref = int(np.searchsorted(c, u * c[-1], side="right"))
        if min(abs(c[max(ref - 1, 0)] - u * c[-1]), abs(c[min(ref, 999)] - u * c[-1])) < 1e-9:
            continue
        assert oracle.categorical(w, u) == ref


def test_categorical_never_selects_zero_weight():
    w = np.array([0.0, 1e-300, 0.0, 0.0, 5.0, 0.0])
    for u in np.linspace(0, 1, 1001, endpoint=False):
        assert w[oracle.categorical(w, u)] > 0


def test_draft_rows_greedy_is_argmax_and_topk():
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, (2, 4, 300)).round(2)
    out = oracle.draft_rows(z, 5, 0.0)
    for b in range(2):
        for g in range(4):
            assert out["draft"][b, g] == np.argmax(z[b, g])
            np.testing.assert_array_equal(out["idx"][b, g],
                                          np.lexsort((np.arange(300), -z[b, g]))[:5])


def test_draft_rows_sampled_is_inverse_cdf_of_softmax():
    rng = np.random.default_rng(4)
    z = rng.normal(0, 2, (3, 8, 1024))
    T = 0.7
    seeds = np.array([11, 12, 13], dtype=np.uint64)
    out = oracle.draft_rows(z, 4, T, seeds=seeds, step=9)
    for b in range(3):
        for g in range(8):
            p = softmax(z[b, g] / T)
            c = np.cumsum(p)
            u = oracle.uniform(int(seeds[b]), 9, b, g, 0)
            ref = int(np.searchsorted(c, u * c[-1], side="right"))
            assert out["draft"][b, g] == ref
            assert abs(out["lse"][b, g] - logsumexp(z[b, g] / T)) < 1e-10


def test_draft_draw_frequencies_follow_softmax():
    z = np.array([[[1.0, 0.0, -1.0, 2.0, 0.5]]])
    T = 0.8
    p = softmax(z[0, 0] / T)
    n = 20000
    counts = np.zeros(5)
    seeds = np.array([7], dtype=np.uint64)
    for s in range(n):
        counts[oracle.draft_rows(z, 1, T, seeds=seeds, step=s)["draft"][0, 0]] += 1
    stat = ((counts - n * p) ** 2 / (n * p)).sum()
    assert stat < chi2.ppf(1 - 1e-6, 4)
