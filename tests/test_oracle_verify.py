"""Pins for the oracle's verification step (CPU only).

"DFlash vs DFlash 2", "The problem: one expensive token at a time": the target
scores the block in one pass, keeps the longest valid prefix and corrects the
first rejection; greedy keeps a draft while it equals the target's choice;
sampling accepts y with probability min(1, p(y)/q(y)), draws a correction from
the residual proportional to [p - q]_+, and emits a bonus token when every
draft survives, so that the committed output is distributed exactly as the
target.  "Beam 1.0 DFlash2", "Evaluation": a block of 8 verifies 7 drafts.

Pins: the textbook greedy rule, exhaustive enumeration of the sampled rule on
tiny vocabularies (the committed-token distribution must equal the target's
product distribution to 1e-12), closed-form special cases, and Monte-Carlo
rates over the Philox uniforms.
"""
import itertools
import zlib

import numpy as np
import pytest
from scipy.special import softmax

import oracle


# ------------------------------------------------------------------ greedy
def _onehot_rows(tokens, V, hot=3.0):
    z = np.zeros((len(tokens), V))
    for r, t in enumerate(tokens):
        z[r, t] = hot
    return z


@pytest.mark.parametrize("targets,drafts,j", [
    ([1, 2, 0, 3], [1, 2, 0], 3),    # all match: tau = gamma, bonus = last argmax
    ([1, 2, 0, 3], [0, 2, 0], 0),    # first mismatch: tau = 1
    ([1, 2, 0, 3], [1, 2, 1], 2),    # mismatch in the middle
    ([1, 2, 0, 3], [1, 0, 0], 1),    # later matches after a mismatch do not count
])
def test_greedy_longest_prefix_then_target_token(targets, drafts, j):
    V = 5
    zp = _onehot_rows(targets, V)
    res = oracle.spec_verify(zp[None], None, np.array([drafts]), 0.0)
    assert res["accept_len"][0] == j
    expect = drafts[:j] + [targets[j]] + [-1] * (len(targets) - j - 1)
    assert res["out_tokens"][0].tolist() == expect
    assert res["accepted"][0].tolist() == [int(d == t) for d, t in zip(drafts, targets)]


def test_greedy_ties_take_lowest_index():
    zp = np.array([[[0.0, 2.0, 2.0, 1.0], [5.0, 5.0, 0.0, 0.0]]])
    res = oracle.spec_verify(zp, None, np.array([[2]]), 0.0)
    assert res["accept_len"][0] == 0 and res["out_tokens"][0].tolist() == [1, -1]
    res = oracle.spec_verify(zp, None, np.array([[1]]), 0.0)
    assert res["accept_len"][0] == 1 and res["out_tokens"][0].tolist() == [1, 0]


def test_greedy_block_of_one_is_plain_argmax():
    zp = np.array([[[0.1, 0.9, 0.3]]])
    res = oracle.spec_verify(zp, None, np.zeros((1, 0), dtype=np.int64), 0.0)
    assert res["accept_len"][0] == 0 and res["out_tokens"][0].tolist() == [1]


# ----------------------------------------------------- sampled: enumeration
def _table_logits(key, V, scale=1.5):
    rng = np.random.default_rng(zlib.crc32(repr(key).encode()))
    return rng.normal(0.0, scale, V)


def _p_target(prefix, V):
    return softmax(_table_logits(("p",) + tuple(prefix), V))


def _q_draft(context, k, V):
    """Drafter distribution of block position k: a function of the context only
    (one parallel pass), not of the other drafts."""
    return softmax(_table_logits(("q", k) + tuple(context), V))


def _cycle(prefix, V, G, T, verify):
    """All outcomes of one draft-verify cycle from `prefix`, with exact probabilities.

    Cells are built from the tables themselves (accept probability min(1, p/q),
    residual cut points), not from anything the oracle computes; u is placed at
    the centre of each cell and the oracle decides."""
    qs = [_q_draft(prefix, k, V) for k in range(G)]
    out = {}
    for drafts in itertools.product(range(V), repeat=G - 1):
        pd = float(np.prod([qs[k][d] for k, d in enumerate(drafts)]))
        ps = [_p_target(tuple(prefix) + drafts[:r], V) for r in range(G)]
        zp = T * np.log(np.array(ps))
        zq = T * np.log(np.array(qs))
        a = [min(1.0, ps[r][drafts[r]] / qs[r][drafts[r]]) for r in range(G - 1)]
        for j in range(G):
            pj = float(np.prod(a[:j])) * ((1.0 - a[j]) if j < G - 1 else 1.0)
            if pj <= 0.0:
                continue
            u_acc = [a[r] / 2 if r < j else ((1.0 + a[r]) / 2 if r == j else 0.5)
                     for r in range(G - 1)]
            if j < G - 1:
                w = np.maximum(ps[j] - qs[j], 0.0)
                if w.sum() <= 0:
                    w = ps[j].copy()
            else:
                w = ps[j].copy()
            c = np.cumsum(w)
            for i in range(V):
                if w[i] <= 0:
                    continue
                u_draw = np.full(G, ((c[i] - w[i]) + c[i]) / 2 / c[-1])
                res = verify(zp, zq, np.array(drafts, dtype=np.int64), T, u_acc, u_draw)
                tau = res["accept_len"] + 1
                committed = tuple(int(t) for t in res["out_tokens"][:tau])
                key = tuple(prefix) + committed
                out[key] = out.get(key, 0.0) + pd * pj * w[i] / c[-1]
    return out


def _committed_distribution(V, G, T, N, verify):
    states = {(): 1.0}
    done = {}
    while states:
        nxt = {}
        for prefix, pr in states.items():
            for key, p2 in _cycle(prefix, V, G, T, verify).items():
                tgt = done if len(key) >= N else nxt
                k2 = key[:N] if len(key) >= N else key
                tgt[k2] = tgt.get(k2, 0.0) + pr * p2
        states = nxt
    return done


def _target_distribution(V, N):
    dist = {}
    for seq in itertools.product(range(V), repeat=N):
        p = 1.0
        for i in range(N):
            p *= _p_target(seq[:i], V)[seq[i]]
        dist[seq] = p
    return dist


def _oracle_verify(zp, zq, drafts, T, u_acc, u_draw):
    return oracle.sampled_verify_seq_u(zp, zq, drafts, T, u_acc, u_draw)


@pytest.mark.parametrize("V,G,N,T", [(3, 3, 3, 0.7), (3, 4, 4, 1.0), (4, 3, 3, 0.7), (2, 5, 5, 1.3)])
def test_sampled_verify_is_lossless_by_enumeration(V, G, N, T):
    got = _committed_distribution(V, G, T, N, _oracle_verify)
    ref = _target_distribution(V, N)
    assert abs(sum(got.values()) - 1.0) < 1e-12
    assert set(got) <= set(ref)
    for seq, p in ref.items():
        assert abs(got.get(seq, 0.0) - p) < 1e-12, (seq, got.get(seq, 0.0), p)


@pytest.mark.parametrize("mistake", ["swap_p_q", "correct_from_next_row", "no_clip"])
def test_enumeration_catches_planted_mistakes(mistake):
    """The enumeration is sensitive: a verifier with a plausible mistake (run on
    the CPU, built around the oracle) does not reproduce the target."""
    def wrong(zp, zq, drafts, T, u_acc, u_draw):
        G = zp.shape[0]
        if mistake == "swap_p_q":
            return oracle.sampled_verify_seq_u(zq, zp, drafts, T, u_acc, u_draw)
        res = oracle.sampled_verify_seq_u(zp, zq, drafts, T, u_acc, u_draw)
        j = res["accept_len"]
        if j < G - 1:
            p = softmax(zp / T, axis=1)
            q = softmax(zq / T, axis=1)
            r = min(j + 1, G - 1) if mistake == "correct_from_next_row" else j
            w = (p[r] - q[r]) if mistake == "no_clip" else np.maximum(p[r] - q[r], 0)
            if mistake == "no_clip":
                w = np.abs(w)
            res["out_tokens"][j] = oracle.categorical(w, u_draw[j])
        return res
    got = _committed_distribution(3, 3, 0.7, 3, wrong)
    ref = _target_distribution(3, 3)
    err = max(abs(got.get(s, 0.0) - p) for s, p in ref.items())
    assert err > 1e-4


# ------------------------------------ sampled with deterministic drafts
def _det_drafts(prefix, V, G):
    """Deterministic drafts (what a selector would produce): a fixed function of the
    context, unrelated to the target."""
    h = zlib.crc32(repr(("sel",) + tuple(prefix)).encode())
    return tuple((h >> (3 * i)) % V for i in range(G - 1))


def _cycle_det(prefix, V, G, T, verify, keep_draft_in_residual=False):
    """All outcomes of one cycle with deterministic drafts (q = point mass at each
    draft), with exact probabilities built from the tables: accept with p(d),
    correct from p without d."""
    drafts = _det_drafts(prefix, V, G)
    ps = [_p_target(tuple(prefix) + drafts[:r], V) for r in range(G)]
    zp = T * np.log(np.array(ps))
    a = [ps[r][drafts[r]] for r in range(G - 1)]
    out = {}
    for j in range(G):
        pj = float(np.prod(a[:j])) * ((1.0 - a[j]) if j < G - 1 else 1.0)
        if pj <= 0.0:
            continue
        u_acc = [a[r] / 2 if r < j else ((1.0 + a[r]) / 2 if r == j else 0.5) for r in range(G - 1)]
        w = ps[j].copy()
        if j < G - 1:
            w[drafts[j]] = 0.0
        c = np.cumsum(w)
        for i in range(V):
            if w[i] <= 0:
                continue
            u_draw = np.full(G, ((c[i] - w[i]) + c[i]) / 2 / c[-1])
            res = verify(zp, None, np.array(drafts, dtype=np.int64), T, u_acc, u_draw)
            tau = res["accept_len"] + 1
            committed = tuple(int(t) for t in res["out_tokens"][:tau])
            key = tuple(prefix) + committed
            out[key] = out.get(key, 0.0) + pj * w[i] / c[-1]
    return out


def _committed_distribution_det(V, G, T, N, verify):
    states = {(): 1.0}
    done = {}
    while states:
        nxt = {}
        for prefix, pr in states.items():
            for key, p2 in _cycle_det(prefix, V, G, T, verify).items():
                tgt = done if len(key) >= N else nxt
                k2 = key[:N] if len(key) >= N else key
                tgt[k2] = tgt.get(k2, 0.0) + pr * p2
        states = nxt
    return done


@pytest.mark.parametrize("V,G,N,T", [(3, 3, 3, 0.7), (4, 4, 4, 1.0), (2, 5, 5, 1.3)])
def test_deterministic_drafts_are_lossless_by_enumeration(V, G, N, T):
    got = _committed_distribution_det(V, G, T, N, _oracle_verify)
    ref = _target_distribution(V, N)
    assert abs(sum(got.values()) - 1.0) < 1e-12
    for seq, p in ref.items():
        assert abs(got.get(seq, 0.0) - p) < 1e-12, (seq, got.get(seq, 0.0), p)


def test_deterministic_enumeration_catches_a_residual_that_keeps_the_draft():
    """A verifier that corrects from p itself (the rejected draft not removed) is
    not lossless, and the enumeration sees it."""
    def wrong(zp, zq, drafts, T, u_acc, u_draw):
        res = oracle.sampled_verify_seq_u(zp, None, drafts, T, u_acc, u_draw)
        j = res["accept_len"]
        if j < zp.shape[0] - 1:
            res["out_tokens"][j] = oracle.categorical(softmax(zp[j] / T), u_draw[j])
        return res
    got = _committed_distribution_det(3, 3, 0.7, 3, wrong)
    ref = _target_distribution(3, 3)
    assert max(abs(got.get(s, 0.0) - p) for s, p in ref.items()) > 1e-4


def test_deterministic_draft_accepted_with_probability_p():
    V = 4
    p = np.array([0.1, 0.6, 0.2, 0.1])
    zp = np.log(p)[None, None, :].repeat(2, 1)
    n = 20000
    res = [oracle.spec_verify(zp, None, np.array([[1]]), 1.0, seeds=np.array([9], np.uint64), step=s)
           for s in range(n)]
    acc = sum(r["accept_len"][0] for r in res)
    sd = np.sqrt(n * 0.6 * 0.4)
    assert abs(acc - n * 0.6) < 5 * sd
    # a rejected draft is never the correction
    assert all(r["out_tokens"][0, 0] != 1 for r in res if r["accept_len"][0] == 0)
    assert np.allclose([r["ratio"][0, 0] for r in res[:3]], 0.6, rtol=1e-12)


# ----------------------------------------------------- sampled: special cases
def test_q_equal_p_accepts_everything():
    rng = np.random.default_rng(0)
    z = rng.normal(0, 1, (1, 5, 7))
    drafts = rng.integers(0, 7, (1, 4))
    for step in range(50):
        res = oracle.spec_verify(z, z, drafts, 0.9, seeds=np.array([3], np.uint64), step=step)
        assert res["accept_len"][0] == 4
        assert res["out_tokens"][0, :4].tolist() == drafts[0].tolist()


def test_disjoint_point_masses_reject_and_correct_to_target():
    V, G = 6, 4
    zp = np.full((1, G, V), -1e4)
    zq = np.full((1, G, V), -1e4)
    zp[0, :, 2] = 0.0
    zq[0, :, 5] = 0.0
    drafts = np.full((1, G - 1), 5)
    for step in range(20):
        res = oracle.spec_verify(zp, zq, drafts, 1.0, seeds=np.array([1], np.uint64), step=step)
        assert res["accept_len"][0] == 0
        assert res["out_tokens"][0].tolist() == [2, -1, -1, -1]


def test_point_mass_proposal_accepts_with_probability_p():
    V = 4
    p = np.array([0.1, 0.6, 0.2, 0.1])
    zp = np.log(p)[None, None, :].repeat(2, 1)
    zq = np.full((1, 2, V), -1e4)
    zq[0, :, 1] = 0.0
    n = 20000
    acc = sum(oracle.spec_verify(zp, zq, np.array([[1]]), 1.0, seeds=np.array([9], np.uint64),
                                 step=s)["accept_len"][0] for s in range(n))
    sd = np.sqrt(n * 0.6 * 0.4)
    assert abs(acc - n * 0.6) < 5 * sd


def test_monte_carlo_accept_rates_and_residual():
    """Drafts from the oracle's own Philox draw; per-position accept rate equals
    sum_v min(p, q); the correction at a rejected first position follows
    [p - q]_+ normalised; E[tau] = 1 + sum_m prod_{k<=m} alpha_k."""
    V, G, T = 5, 4, 1.0
    rng = np.random.default_rng(5)
    zt = rng.normal(0, 1.0, (1, G, V))
    zd = zt + rng.normal(0, 1.0, (1, G, V))
    p = softmax(zt[0] / T, axis=1)
    q = softmax(zd[0] / T, axis=1)
    alpha = np.minimum(p, q).sum(1)
    resid0 = np.maximum(p[0] - q[0], 0)
    resid0 /= resid0.sum()
    n = 12000
    seeds = np.array([17], np.uint64)
    acc = np.zeros(G - 1)
    taus = []
    corr = np.zeros(V)
    for s in range(n):
        d = oracle.draft_rows(zd, 1, T, seeds=seeds, step=s)["draft"][:, :G - 1]
        res = oracle.spec_verify(zt, zd, d, T, seeds=seeds, step=s)
        acc += res["accepted"][0]
        taus.append(res["accept_len"][0] + 1)
        if res["accept_len"][0] == 0:
            corr[res["out_tokens"][0, 0]] += 1
    for r in range(G - 1):
        sd = np.sqrt(n * alpha[r] * (1 - alpha[r]))
        assert abs(acc[r] - n * alpha[r]) < 5 * sd
    e_tau = 1 + sum(np.prod(alpha[:m]) for m in range(1, G))
    assert abs(np.mean(taus) - e_tau) < 5 * np.std(taus) / np.sqrt(n)
    m = corr.sum()
    mask = resid0 > 0
    stat = ((corr[mask] - m * resid0[mask]) ** 2 / (m * resid0[mask])).sum()
    assert corr[~mask].sum() == 0
    from scipy.stats import chi2
    assert stat < chi2.ppf(1 - 1e-6, mask.sum() - 1)


def test_verify_uses_documented_counters():
    """Accept test of row r uses purpose 1 at (step, b, r); the draw at row j uses
    purpose 2 at (step, b, j)."""
    V, G, T = 50, 4, 0.8
    rng = np.random.default_rng(8)
    zt = rng.normal(0, 2, (2, G, V))
    zd = zt + rng.normal(0, 1, (2, G, V))
    drafts = rng.integers(0, V, (2, G - 1))
    seeds = np.array([4, 5], np.uint64)
    res = oracle.spec_verify(zt, zd, drafts, T, seeds=seeds, step=3)
    for b in range(2):
        ua = [oracle.uniform(int(seeds[b]), 3, b, r, 1) for r in range(G - 1)]
        ud = [oracle.uniform(int(seeds[b]), 3, b, r, 2) for r in range(G)]
        one = oracle.sampled_verify_seq_u(zt[b], zd[b], drafts[b], T, ua, ud)
        assert one["accept_len"] == res["accept_len"][b]
        assert one["out_tokens"].tolist() == res["out_tokens"][b].tolist()


def test_draft_with_zero_target_and_draft_probability_is_rejected():
    """A draft that neither p nor q can produce (both logits -inf there, as for
    a draft outside a truncated row) makes p/q = 0/0.  The target gives it no
    probability, so committing it would leave the target's distribution: it is
    rejected for every uniform, and the correction is drawn from [p - q]_+."""
    V, G, T = 5, 3, 1.0
    zp = np.log(np.array([[0.5, 0.5, 0.0, 0.0, 0.0]] * G))
    zq = np.log(np.array([[0.25, 0.25, 0.0, 0.5, 0.0]] * G))
    drafts = np.array([[2, 2]])
    for step in range(200):
        res = oracle.spec_verify(zp[None], zq[None], drafts, T, seeds=np.array([6], np.uint64),
                                 step=step)
        assert res["accept_len"][0] == 0
        assert res["accepted"][0].tolist() == [0, 0]
        assert res["out_tokens"][0, 0] in (0, 1)   # the residual's support
    assert np.isnan(res["ratio"][0, 0])
    # with u fixed at 0 (the most permissive uniform) the draft is still rejected
    one = oracle.sampled_verify_seq_u(zp, zq, drafts[0], T, [0.0, 0.0], [0.3, 0.3, 0.3])
    assert one["accept_len"] == 0 and one["accepted"].tolist() == [0, 0]
