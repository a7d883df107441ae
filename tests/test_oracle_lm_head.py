"""Pins for the oracle's drafter LM head (CPU only).

The drafter reuses the target's LM head ("Beam 1.0 DFlash2" model card,
"Model"); top-k per position follows "DFlash vs DFlash 2", "The candidate
selector"; the draft is a draw from q = softmax(z/T) ("The problem: one
expensive token at a time"), made in two inverse-CDF steps over 128-entry
vocabulary segments.  Pins: numpy matmul (library) for the logits, numpy
lexsort / argmax and scipy logsumexp (library) for top-k and the normaliser,
numpy's Philox and searchsorted (library) for each draw step on inputs where
the other step is forced, a chi-square check that the two steps together
sample softmax(z/T) exactly, and the row-subset invariant.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax
from scipy.stats import chi2

import oracle

MASK64 = (1 << 64) - 1
SEG = 128


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


def test_one_segment_draw_is_the_inverse_cdf():
    """V <= 128: the segment step always picks segment 0, so the draft is the
    inverse CDF of softmax(z/T) at the uniform of purpose 3."""
    h, w = inputs(24, 32, 100, 3, w_std=0.4)
    z = bits_to_f64(h) @ bits_to_f64(w).T
    G, T, step = 8, 0.7, 11
    seeds = np.array([5, 9, 13], dtype=np.uint64)
    r = oracle.lm_head_topk(h, w, G, 4, T, seeds=seeds, step=step)
    for i in range(24):
        b, g = divmod(i, G)
        p = softmax(z[i] / T)
        u = np_uniform(int(seeds[b]), step, b, g, 3)
        assert r["draft"][i] == np.searchsorted(np.cumsum(p), u * p.sum(), side="right")


def test_segment_step_picks_segments_by_mass():
    """One dominant entry per 128-entry segment (every other logit 60 below):
    the draft is the dominant entry of the segment the purpose-0 uniform picks
    by the inverse CDF of the segment masses.  The last segment is ragged."""
    V = 5 * SEG + 40
    dom = np.array([7, 130, 300, 385, 600, 650])       # one per segment
    logm = np.array([0.5, -1.0, 1.25, 0.0, 2.0, -0.5])  # bf16-exact log-masses
    zcol = np.full(V, -60.0)
    zcol[dom] = logm
    h, w = one_hot_head(zcol, 40)
    T = 1.0
    seeds = np.arange(40, dtype=np.uint64) * 3 + 1
    r = oracle.lm_head_topk(h, w, 1, 2, T, seeds=seeds, step=4)
    mass = np.exp(logm)
    cum = np.cumsum(mass) / mass.sum()
    for i in range(40):
        J = np.searchsorted(cum, np_uniform(int(seeds[i]), 4, i, 0, 0), side="right")
        assert r["draft"][i] == dom[J]


def test_entry_step_uses_the_segment_uniform():
    """All mass in segment J (the rest 60 below): the draft is the inverse CDF
    inside J at the uniform of purpose 3 + 256 J."""
    V = 6 * SEG
    rng = np.random.default_rng(4)
    for J in (1, 4, 5):
        zcol = np.full(V, -60.0)
        zcol[J * SEG:(J + 1) * SEG] = bits_to_f64(bf16_bits(rng.standard_normal(SEG)))
        h, w = one_hot_head(zcol, 16)
        T = 0.8
        r = oracle.lm_head_topk(h, w, 4, 3, T, seeds=np.arange(4) + 100, step=2)
        p = softmax(zcol[J * SEG:(J + 1) * SEG] / T)
        for i in range(16):
            b, g = divmod(i, 4)
            u = np_uniform(100 + b, 2, b, g, 3 + 256 * J)
            assert r["draft"][i] == J * SEG + np.searchsorted(np.cumsum(p), u * p.sum(),
                                                              side="right")


def test_two_step_draw_samples_softmax():
    """Many rows with the same logits and distinct counters: the draft
    frequencies match softmax(z/T) over a ragged three-segment vocabulary."""
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
    # per-segment totals agree too (the segment step alone)
    seg_obs = np.add.reduceat(counts, [0, SEG, 2 * SEG])
    seg_p = np.add.reduceat(p, [0, SEG, 2 * SEG])
    assert np.all(np.abs(seg_obs - seg_p * n) < 5 * np.sqrt(n * seg_p * (1 - seg_p)) + 1)


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
