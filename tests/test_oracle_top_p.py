"""Pins for the oracle's top-p (nucleus) truncation (CPU only).

"Beam 1.0 DFlash2" model card, "Evaluation": sampled runs use temperature 0.7
and top-p 0.99.  The nucleus of softmax(z/T) is the shortest prefix, in the
order (logit descending, index ascending), whose probability reaches top_p;
masking the rest to -inf makes softmax(z/T) the renormalised truncation, and
"DFlash vs DFlash 2", "The problem: one expensive token at a time": verifying
drafts drawn from the drafter's truncation against the target's truncation
commits tokens distributed exactly as the truncated target.

Pins: the three properties that characterise the nucleus (its mass reaches
top_p, dropping its last entry falls short, and it is a prefix of the rank
order), checked with numpy / scipy on random rows with ties; closed forms
(equal logits, top_p >= 1, a tiny top_p); and exhaustive enumeration of the
oracle's sampled verification run on masked rows.
"""
import itertools
import zlib

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def rank_order(z):
    return np.lexsort((np.arange(len(z)), -z))


@pytest.mark.parametrize("T,top_p", [(0.7, 0.99), (1.0, 0.9), (0.5, 0.5), (1.3, 0.999)])
def test_nucleus_properties(T, top_p):
    rng = np.random.default_rng(zlib.crc32(repr((T, top_p)).encode()))
    z = rng.standard_normal((12, 400)) * 2.0
    z[3] = np.round(z[3])                      # many exact ties
    z[5, :40] = z[5].max()                     # a tied block of maxima
    out, kept = oracle.top_p_mask(z, T, top_p)
    for r in range(z.shape[0]):
        p = softmax(z[r] / T)
        keep = np.isfinite(out[r])
        assert keep.sum() == kept[r]
        np.testing.assert_array_equal(out[r][keep], z[r][keep])
        order = rank_order(z[r])
        K = int(kept[r])
        # a prefix of the rank order
        assert keep[order[:K]].all() and not keep[order[K:]].any()
        mass = p[order[:K]].sum()
        assert mass >= top_p - 1e-12
        if K > 1:
            assert mass - p[order[K - 1]] < top_p + 1e-12   # dropping the last falls short


def test_equal_logits_keep_the_lowest_indices():
    z = np.full((2, 64), 1.5)
    out, kept = oracle.top_p_mask(z, 0.7, 0.75)     # 48 of 64 equal entries (exact in binary)
    assert kept.tolist() == [48, 48]
    assert np.isfinite(out[:, :48]).all() and np.isinf(out[:, 48:]).all()


def test_top_p_one_keeps_everything_and_tiny_top_p_keeps_the_argmax():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((4, 300))
    z[1, [10, 200]] = z[1].max() + 1.0              # tied maximum: the lower index is kept
    out, kept = oracle.top_p_mask(z, 0.7, 1.0)
    np.testing.assert_array_equal(out, z)
    assert (kept == 300).all()
    out, kept = oracle.top_p_mask(z, 0.7, 1e-9)
    assert (kept == 1).all()
    for r in range(4):
        assert np.argmax(np.isfinite(out[r])) == np.argmax(z[r]) and np.isfinite(out[r]).sum() == 1


def keep_rule(z, logit, index):
    """The cut's membership rule: z_v > logit, or z_v == logit and v <= index."""
    v = np.arange(z.shape[-1])
    return (z > logit) | ((z == logit) & (v <= index))


@pytest.mark.parametrize("T,top_p", [(0.7, 0.99), (1.0, 0.9), (0.5, 0.5), (0.7, 1.0), (0.7, 1e-9)])
def test_cut_names_the_nucleus(T, top_p):
    """The cut (last nucleus entry in rank order) reproduces the mask through
    the membership rule, on rows with exact ties, a tied block of maxima,
    signed zeros and -inf entries; the nucleus is the first `kept` entries of
    numpy's rank order."""
    rng = np.random.default_rng(zlib.crc32(repr(("cut", T, top_p)).encode()))
    z = rng.standard_normal((10, 500)) * 2.0
    z[2] = np.round(z[2])
    z[4, :30] = z[4].max()
    z[6, 100:300] = -np.inf
    z[7, ::2] = 0.0
    z[7, 1::2] = -0.0                               # equal values: ranked by index alone
    out, kept = oracle.top_p_mask(z, T, top_p)
    logit, index, kept2 = oracle.top_p_cut(z, T, top_p)
    np.testing.assert_array_equal(kept2, kept)
    for r in range(z.shape[0]):
        keep = keep_rule(z[r], logit[r], index[r])
        assert keep.sum() == kept[r]
        first = np.zeros(z.shape[1], dtype=bool)
        first[rank_order(z[r])[:kept[r]]] = True
        np.testing.assert_array_equal(keep, first)
        np.testing.assert_array_equal(out[r], np.where(keep, z[r], -np.inf))


def test_cut_closed_forms():
    z = np.array([[3.0, 2.0, 1.0, 0.0, -1.0], [1.0, 5.0, 5.0, 0.5, 5.0]])
    logit, index, kept = oracle.top_p_cut(z, 1.0, 0.9)   # row 0: 0.636, 0.870, 0.956 -> 3 kept
    assert (logit[0], index[0], kept[0]) == (1.0, 2, 3)
    logit, index, kept = oracle.top_p_cut(z, 1.0, 1e-9)  # the argmax, lowest index among ties
    assert (logit[1], index[1], kept[1]) == (5.0, 1, 1)
    logit, index, kept = oracle.top_p_cut(z, 1.0, 1.0)   # everything: the last entry in rank order
    assert (logit[0], index[0]) == (-1.0, 4) and (logit[1], index[1]) == (0.5, 3)
    assert (kept == 5).all()


def test_masking_is_temperature_dependent_as_defined():
    z = np.array([[3.0, 2.0, 1.0, 0.0, -1.0]])
    # T = 1: p = (0.636, 0.234, 0.086, 0.032, 0.012); cumulative 0.636, 0.870, 0.956
    out, kept = oracle.top_p_mask(z, 1.0, 0.9)
    assert kept[0] == 3 and np.isinf(out[0, 3:]).all()
    # T = 2 flattens it: p = (0.429, 0.260, 0.158, 0.096, 0.058); cumulative 0.846, then 0.942
    out, kept = oracle.top_p_mask(z, 2.0, 0.9)
    assert kept[0] == 4 and np.isinf(out[0, 4])


# --------------------------------------- verification of truncated tables
def _table(key, V, scale=1.5):
    rng = np.random.default_rng(zlib.crc32(repr(key).encode()))
    return rng.normal(0.0, scale, V)


def _trunc(logits, T, top_p):
    zm, _ = oracle.top_p_mask(logits[None], T, top_p)
    return softmax(zm[0] / T)


def _p(prefix, V, T, top_p):
    return _trunc(_table(("p",) + tuple(prefix), V), T, top_p)


def _q(context, k, V, T, top_p):
    return _trunc(_table(("q", k) + tuple(context), V), T, top_p)


def _cycle(prefix, V, G, T, top_p):
    """All outcomes of one cycle with exact probabilities: drafts from the
    drafter's truncation, the oracle's verification on masked rows (logit
    T log p', -inf outside the nucleus), u at the centre of each decision cell."""
    qs = [_q(prefix, k, V, T, top_p) for k in range(G)]
    out = {}
    with np.errstate(divide="ignore"):
        zq = T * np.log(np.array(qs))
    for drafts in itertools.product(range(V), repeat=G - 1):
        pd = float(np.prod([qs[k][d] for k, d in enumerate(drafts)]))
        if pd <= 0.0:
            continue
        ps = [_p(tuple(prefix) + drafts[:r], V, T, top_p) for r in range(G)]
        with np.errstate(divide="ignore"):
            zp = T * np.log(np.array(ps))
        a = [min(1.0, ps[r][drafts[r]] / qs[r][drafts[r]]) for r in range(G - 1)]
        for j in range(G):
            pj = float(np.prod(a[:j])) * ((1.0 - a[j]) if j < G - 1 else 1.0)
            if pj <= 0.0:
                continue
            u_acc = [a[r] / 2 if r < j else ((1.0 + a[r]) / 2 if r == j else 0.5)
                     for r in range(G - 1)]
            w = np.maximum(ps[j] - qs[j], 0.0) if j < G - 1 else ps[j].copy()
            if w.sum() <= 0:
                w = ps[j].copy()
            c = np.cumsum(w)
            for i in range(V):
                if w[i] <= 0:
                    continue
                u_draw = np.full(G, ((c[i] - w[i]) + c[i]) / 2 / c[-1])
                res = oracle.sampled_verify_seq_u(zp, zq, np.array(drafts, dtype=np.int64), T,
                                                  u_acc, u_draw)
                tau = res["accept_len"] + 1
                key = tuple(prefix) + tuple(int(t) for t in res["out_tokens"][:tau])
                out[key] = out.get(key, 0.0) + pd * pj * w[i] / c[-1]
    return out


@pytest.mark.parametrize("V,G,N,T,top_p", [(4, 3, 3, 0.7, 0.8), (5, 3, 3, 1.0, 0.7), (4, 4, 3, 0.7, 0.95)])
def test_verification_of_truncated_rows_is_lossless(V, G, N, T, top_p):
    states, done = {(): 1.0}, {}
    while states:
        nxt = {}
        for prefix, pr in states.items():
            for key, p2 in _cycle(prefix, V, G, T, top_p).items():
                tgt = done if len(key) >= N else nxt
                k2 = key[:N] if len(key) >= N else key
                tgt[k2] = tgt.get(k2, 0.0) + pr * p2
        states = nxt
    ref = {}
    for seq in itertools.product(range(V), repeat=N):
        pr = 1.0
        for i in range(N):
            pr *= _p(seq[:i], V, T, top_p)[seq[i]]
        if pr > 0:
            ref[seq] = pr
    assert abs(sum(done.values()) - 1.0) < 1e-12
    assert set(done) <= set(ref)                 # nothing outside the target's nuclei
    for seq, pr in ref.items():
        assert abs(done.get(seq, 0.0) - pr) < 1e-12, (seq, done.get(seq, 0.0), pr)
