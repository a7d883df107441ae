"""Pins for the oracle's drafter LM head (CPU only).

The drafter reuses the target's LM head ("Beam 1.0 DFlash2" model card,
"Model"); top-k per position follows "DFlash vs DFlash 2", "The candidate
selector"; the draft is a draw from q = softmax(z/T) ("The problem: one
expensive token at a time"), one inverse-CDF draw over the whole row in
increasing vocabulary order at the row's purpose-0 uniform.  Pins: numpy
matmul (library) for the logits, numpy lexsort / argmax and scipy logsumexp
(library) for top-k and the normaliser, numpy's Philox and searchsorted
(library) for the draw, a chi-square check that the draws sample
softmax(z/T), and the row-subset invariant.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax
from scipy.stats import chi2

import oracle

MASK64 = (1 << 64) - 1


def bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def np_uniform(seed, step, b, row, purpose):
    c = [step, b, row, purpose]
    v = (sum(int(w) << (64 * i) for i, w in enumerate(c)) - 1) & ((1 << 256) - 1)
    ctr = np.array([(v >> (64 * i)) & MASK64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=ctr, key=np.array([seed, 0], dtype=np.uint64))
    return (int(bg.random_raw(4)[0]) >> 11) * 2.0 ** -53


def inputs(n, d, V, seed, w_std=0.3):
    rng = np.random.default_rng(seed)
    h = bf16_bits(rng.standard_normal((n, d)))
    w = bf16_bits(rng.standard_normal((V, d)) * w_std)
    return h, w


def one_hot_head(zcol, n):
    """h = e_0 and W[:, 0] = z: the logits are exactly the bf16 values zcol."""
    V = len(zcol)
    h = np.zeros((n, 8), dtype=np.float32)
    h[:, 0] = 1.0
    w = np.zeros((V, 8), dtype=np.float32)
    w[:, 0] = zcol
    return bf16_bits(h), bf16_bits(w)


def test_logits_are_the_matmul():
    h, w = inputs(5, 96, 333, 1)
    r = oracle.lm_head_topk(h, w, 5, 4, 0.7, seeds=np.arange(1), want_z=True)
    ref = bits_to_f64(h) @ bits_to_f64(w).T
    np.testing.assert_allclose(r["z"], ref, rtol=1e-12, atol=1e-12)


def test_topk_lse_and_greedy_match_library_routines():
    h, w = inputs(6, 64, 700, 2)
    w[10] = w[500]                                   # exact logit tie: lower index ranks first
    z = bits_to_f64(h) @ bits_to_f64(w).T
    for T in (0.7, 1.0):
        r = oracle.lm_head_topk(h, w, 3, 9, T, seeds=np.arange(2), step=1)
        for i in range(6):
            order = np.lexsort((np.arange(700), -z[i]))[:9]
            np.testing.assert_array_equal(r["idx"][i], order)
            np.testing.assert_array_equal(r["val"][i], z[i][order])
        np.testing.assert_allclose(r["lse"], logsumexp(z / T, axis=1), rtol=0, atol=1e-12)
    g = oracle.lm_head_topk(h, w, 3, 9, 0.0)
    assert np.isnan(g["lse"]).all()
    np.testing.assert_array_equal(g["draft"], np.argmax(z, axis=1))
    np.testing.assert_array_equal(g["draft"], g["idx"][:, 0])


def test_draw_is_the_inverse_cdf_over_the_row():
    """The draft is the smallest index whose cumulative softmax(z/T) mass (in
    increasing vocabulary order) exceeds u times the total, u the purpose-0
    uniform of (seed, step, sequence, block row): numpy's Philox and
    searchsorted, over rows of several hundred entries."""
    h, w = inputs(24, 32, 700, 3, w_std=0.4)
    z = bits_to_f64(h) @ bits_to_f64(w).T
    G, T, step = 8, 0.7, 11
    seeds = np.array([5, 9, 13], dtype=np.uint64)
    r = oracle.lm_head_topk(h, w, G, 4, T, seeds=seeds, step=step)
    for i in range(24):
        b, g = divmod(i, G)
        p = softmax(z[i] / T)
        u = np_uniform(int(seeds[b]), step, b, g, 0)
        assert r["draft"][i] == np.searchsorted(np.cumsum(p), u * p.sum(), side="right")


def test_draw_on_exact_logits_picks_by_mass():
    """Exact logits (a one-hot hidden row reads one bf16 column of W): six
    dominant entries spread over a 700-entry row, everything else 60 below; the
    draft is the dominant entry whose cumulative mass first exceeds u."""
    V = 700
    dom = np.array([7, 130, 300, 385, 600, 650])
    logm = np.array([0.5, -1.0, 1.25, 0.0, 2.0, -0.5])  # bf16-exact log-masses
    zcol = np.full(V, -60.0)
    zcol[dom] = logm
    h, w = one_hot_head(zcol, 40)
    seeds = np.arange(40, dtype=np.uint64) * 3 + 1
    r = oracle.lm_head_topk(h, w, 1, 2, 1.0, seeds=seeds, step=4)
    mass = np.exp(logm)
    cum = np.cumsum(mass) / mass.sum()
    for i in range(40):
        J = np.searchsorted(cum, np_uniform(int(seeds[i]), 4, i, 0, 0), side="right")
        assert r["draft"][i] == dom[J]


def test_same_draft_as_the_logits_row_draw():
    """Sampling from the LM head's logits is the logits-row draw of dflash_topk's
    definition: with the same seeds and counters both give the same token."""
    h, w = inputs(16, 40, 900, 8)
    z = bits_to_f64(h) @ bits_to_f64(w).T
    seeds = np.array([21, 22], dtype=np.uint64)
    r = oracle.lm_head_topk(h, w, 8, 3, 0.8, seeds=seeds, step=5)
    d = oracle.draft_rows(z.reshape(2, 8, 900), 3, 0.8, seeds=seeds, step=5)
    np.testing.assert_array_equal(r["draft"], d["draft"].reshape(-1))
    np.testing.assert_array_equal(r["idx"], d["idx"].reshape(16, 3))


def test_draw_samples_softmax():
    """Many rows with the same logits and distinct counters: the draft
    frequencies match softmax(z/T) (chi-square)."""
    V, d, n, T = 300, 16, 60000, 0.9
    rng = np.random.default_rng(5)
    h1 = bf16_bits(rng.standard_normal((1, d)))
    w = bf16_bits(rng.standard_normal((V, d)) * 0.35)
    h = np.repeat(h1, n, axis=0)
    r = oracle.lm_head_topk(h, w, 1, 1, T, seeds=np.full(n, 17, dtype=np.uint64), step=0)
    z = (bits_to_f64(h1) @ bits_to_f64(w).T)[0]
    p = softmax(z / T)
    counts = np.bincount(r["draft"], minlength=V)
    exp_ = p * n
    # pool the bins expected below 5 so every cell of the statistic is valid
    small = exp_ < 5
    obs = np.append(counts[~small], counts[small].sum())
    ex = np.append(exp_[~small], exp_[small].sum())
    stat = ((obs - ex) ** 2 / ex).sum()
    assert stat < chi2.ppf(1 - 1e-6, len(obs) - 1), stat


def test_row_subset_matches_full_rows():
    h, w = inputs(16, 48, 500, 6)
    seeds = np.array([3, 1, 4, 1], dtype=np.uint64)
    full = oracle.lm_head_topk(h, w, 4, 5, 0.7, seeds=seeds, step=9)
    pick = np.array([2, 13])
    sub = oracle.lm_head_topk(h[pick], w, 4, 5, 0.7, seeds=seeds, step=9, row_id=pick)
    for key in ("idx", "val", "lse", "draft"):
        np.testing.assert_array_equal(sub[key], full[key][pick])


def test_rejects_bad_arguments():
    h, w = inputs(2, 16, 40, 7)
    with pytest.raises(ValueError):
        oracle.lm_head_topk(h, w, 1, 41, 0.7, seeds=np.arange(2))   # k > V
    with pytest.raises(ValueError):
        oracle.lm_head_topk(h, w, 1, 4, -1.0, seeds=np.arange(2))
    with pytest.raises(ValueError):
        oracle.lm_head_topk(h, w, 1, 4, 0.7)                         # sampling needs seeds
    oracle.lm_head_topk(h, w, 1, 4, 0.7, want_draft=False)          # no draft: no seeds needed
