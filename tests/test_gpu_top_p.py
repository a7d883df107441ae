"""GPU parity of dflash_top_p_mask (top-p nucleus masking) against the fp64
oracle, and of sampling / verification on masked rows (C ABI).

Bar: the GPU's kept set is a prefix of the rank order (logit descending, index
ascending) and equals the oracle's nucleus, except that its size may differ
where the oracle's cumulative probability at the boundary is within 1e-5 of
top_p (the GPU sums fp32 weights in fixed point at 2^-40 of the maximum's).
Kept entries are copied bit-exactly; kept counts equal the finite entries;
in-place masking equals out-of-place.  Verification and draws on masked rows
follow the bar of the unmasked tests (test_gpu_topk_verify.py), with the
oracle run on the oracle's own masks.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
import block_drafting_context_amd as dfl
from block_drafting_context_amd import synthetic as syn
from parity_util import cuda, draw_boundary_ok, to64

pytestmark = pytest.mark.gpu
EPS = 1e-5


def f32(x):
    return float(np.float32(x))


def check_mask(z, T, top_p, what=""):
    print(f"[top_p] {what} rows={z.shape[0]} V={z.shape[1]} T={T} top_p={top_p}", flush=True)
    dev = cuda()
    zg = z.to(dev)
    out, kept = dfl.dflash_top_p_mask(zg, T, top_p, want_kept=True)
    inplace = zg.clone()
    dfl.dflash_top_p_mask(inplace, T, top_p, out=inplace)
    torch.cuda.synchronize()
    got = to64(out)
    np.testing.assert_array_equal(to64(inplace), got)
    z64 = to64(z)
    ref, kref = oracle.top_p_mask(z64, f32(T), f32(top_p))
    kept = to64(kept)
    for r in range(z.shape[0]):
        K, Kr = int(kept[r]), int(kref[r])
        if K == Kr:
            np.testing.assert_array_equal(got[r], ref[r])   # the same nucleus, copied bit-exactly
            continue
        # sizes differ: the GPU's set must still be the first K entries of the rank order,
        # and every cumulative mass between the two boundaries within EPS of top_p
        order = np.lexsort((np.arange(z.shape[1]), -z64[r]))
        fin = np.isfinite(z64[r][order])
        np.testing.assert_array_equal(got[r][order[:K]], z64[r][order[:K]])
        assert np.isneginf(got[r][order[K:]]).all(), (r, "not a prefix")
        p = softmax(z64[r] / f32(T))
        c = np.cumsum(p[order])
        lo, hi = min(K, Kr), max(K, Kr)
        assert fin[:hi].all() and np.all(np.abs(c[lo - 1:hi] - f32(top_p)) < EPS), (r, K, Kr)
    return out


def test_small_rows_with_ties():
    z = syn.normal((12, 3000), 1, "topp_small", std=2.0)
    z[3] = torch.round(z[3])
    z[5, :40] = z[5].max()
    for T, p in ((0.7, 0.99), (1.0, 0.9), (0.5, 0.5), (1.3, 0.999)):
        check_mask(z, T, p, what="small")


def test_equal_logits_overflow_the_gather():
    """65,536 equal logits: one bin holds everything, so the set is narrowed by
    the rank key's digits; the nucleus is the lowest indices."""
    z = torch.full((2, 65536), 0.75)
    out = check_mask(z, 0.7, 0.75, what="equal")
    got = to64(out)
    assert np.isfinite(got[:, :49152]).all() and np.isinf(got[:, 49152:]).all()


def test_edge_top_p_values_and_neg_inf_entries():
    z = syn.normal((4, 5000), 2, "topp_edge", std=2.0)
    z[2, 1000:3000] = -float("inf")
    out = check_mask(z, 0.7, 1.0, what="top_p=1")
    np.testing.assert_array_equal(to64(out), to64(z))
    out = check_mask(z, 0.7, 1e-6, what="tiny")
    assert (np.isfinite(to64(out)).sum(1) == 1).all()
    check_mask(z, 0.7, 0.99, what="-inf entries")


def test_full_vocabulary_rows():
    zt, zd = syn.logits_pair(32, 8, 151936, 2.0, 1.0, seed=3)
    rows = zt.reshape(-1, 151936)
    pick = torch.tensor([0, 17, 40, 63, 77, 90, 111, 128, 130, 151, 170, 191, 200, 223, 240, 255])
    print("[top_p] full vocabulary, 256 rows (oracle on 16)", flush=True)
    dev = cuda()
    out, kept = dfl.dflash_top_p_mask(rows.to(dev), 0.7, 0.99, want_kept=True)
    torch.cuda.synchronize()
    assert (to64(kept) == np.isfinite(to64(out)).sum(1)).all()
    check_mask(rows[pick].contiguous(), 0.7, 0.99, what="full V sample")


def test_sampling_and_verification_on_masked_rows():
    """Top-p decoding: the drafter samples from its truncation (dflash_topk on
    masked drafter rows) and spec_verify checks against the target's truncation
    (masked target rows).  The GPU's masks must equal the oracle's; the draws
    and verification on the masked rows then meet the unmasked bar."""
    from test_gpu_topk_verify import _topk_case, _verify_case
    B, G, V, T, P = 4, 8, 5000, 0.7, 0.9
    zt, zd = syn.logits_pair(B, G, V, 2.0, 1.0, seed=4)
    dev = cuda()
    mt, _ = dfl.dflash_top_p_mask(zt.to(dev), T, P)
    md, _ = dfl.dflash_top_p_mask(zd.to(dev), T, P)
    torch.cuda.synchronize()
    rt, _ = oracle.top_p_mask(to64(zt), f32(T), f32(P))
    rd, _ = oracle.top_p_mask(to64(zd), f32(T), f32(P))
    np.testing.assert_array_equal(to64(mt), rt)
    np.testing.assert_array_equal(to64(md), rd)
    zt_m = torch.from_numpy(rt.astype(np.float32))
    zd_m = torch.from_numpy(rd.astype(np.float32))
    seeds = syn.philox_seeds(B, 3)
    for step in range(3):
        tk = _topk_case(zd_m, 8, T, seeds, step=step, what=f"masked drafter rows {step}")
        drafts = to64(tk["draft"])[:, :G - 1]
        assert np.isfinite(np.take_along_axis(rd[:, :G - 1], drafts[..., None], -1)).all()
        _verify_case(zt_m, zd_m, torch.from_numpy(drafts.astype(np.int64)), T, seeds, step=step,
                     what=f"masked rows {step}")


# ---------------------------------------------------------------- nucleus cuts
def keep_rule(z, logit, index):
    v = np.arange(z.shape[-1])
    return (z > logit) | ((z == logit) & (v <= index))


def check_cut(z, T, top_p, what=""):
    """dflash_top_p_cut: the cut's nucleus (membership rule on the unmasked
    row) has `kept` entries, is what dflash_top_p_mask keeps, and meets the
    mask's bar against the oracle's nucleus."""
    print(f"[top_p cut] {what} rows={z.shape[0]} V={z.shape[1]} T={T} top_p={top_p}", flush=True)
    dev = cuda()
    zg = z.to(dev)
    cut, kept = dfl.dflash_top_p_cut(zg, T, top_p, want_kept=True)
    masked, kept_m = dfl.dflash_top_p_mask(zg, T, top_p, want_kept=True)
    torch.cuda.synchronize()
    lg, ix = (to64(t) for t in dfl.nucleus_cut_values(cut))
    kept, kept_m, got_m = to64(kept), to64(kept_m), to64(masked)
    z64 = to64(z)
    ref, kref = oracle.top_p_mask(z64, f32(T), f32(top_p))
    for r in range(z.shape[0]):
        keep = keep_rule(z64[r], lg[r], ix[r])
        assert keep.sum() == kept[r] == kept_m[r], (r, keep.sum(), kept[r], kept_m[r])
        np.testing.assert_array_equal(got_m[r], np.where(keep, z64[r], -np.inf))
        K, Kr = int(kept[r]), int(kref[r])
        order = np.lexsort((np.arange(z.shape[1]), -z64[r]))
        first = np.zeros(z.shape[1], dtype=bool)
        first[order[:K]] = True
        np.testing.assert_array_equal(keep, first)            # a prefix of the rank order
        if K != Kr:
            p = softmax(z64[r] / f32(T))
            c = np.cumsum(p[order])
            lo, hi = min(K, Kr), max(K, Kr)
            assert np.all(np.abs(c[lo - 1:hi] - f32(top_p)) < EPS), (r, K, Kr)
    return cut


def test_cut_small_rows_ties_and_edges():
    z = syn.normal((12, 3000), 1, "topp_small", std=2.0)
    z[3] = torch.round(z[3])
    z[5, :40] = z[5].max()
    for T, p in ((0.7, 0.99), (1.0, 0.9), (0.5, 0.5), (1.3, 0.999)):
        check_cut(z, T, p, what="small")
    z = syn.normal((4, 5000), 2, "topp_edge", std=2.0)
    z[2, 1000:3000] = -float("inf")
    cut = check_cut(z, 0.7, 1.0, what="top_p=1")
    lg, ix = dfl.nucleus_cut_values(cut.cpu())
    assert torch.isneginf(lg).all() and (ix == 2**31 - 1).all()   # keeps everything
    check_cut(z, 0.7, 1e-6, what="tiny")
    check_cut(z, 0.7, 0.99, what="-inf entries")


def test_cut_equal_logits_and_signed_zeros():
    """65,536 equal logits (the narrowing path); rows of +0.0 and -0.0, which
    rank as equal values, by index."""
    check_cut(torch.full((2, 65536), 0.75), 0.7, 0.75, what="equal")
    z = torch.zeros((3, 4000))
    z[:, 1::2] = -0.0
    z[1, :100] = 2.0
    z[2] = syn.normal((1, 4000), 9, "topp_zero", std=1.0)[0]
    z[2, 500:1500:2] = 0.0
    z[2, 501:1500:2] = -0.0
    for p in (0.3, 0.77, 0.99):
        check_cut(z, 0.7, p, what="signed zeros")


def test_cut_paths_the_sample_does_not_predict():
    """The cut kernel takes its histogram's reference from the first entries
    of the row (every thread's first loads, 32,768 entries).  Rows where that
    sample misleads give the same result through the other paths: a maximum
    far beyond the sample (the histogram is rebuilt relative to it), a sample
    distributed unlike the rest (higher or lower, tied values outside it),
    and a row length that is not a multiple of 4 (no 16-byte loads)."""
    V = 40000
    z = syn.normal((6, V), 11, "topp_paths", std=2.0)
    z[0, V - 3] = 60.0                        # far above the sample's maximum
    z[1, 33000:] += 3.0                        # the unsampled part sits higher
    z[2, :32768] -= 4.0                        # the sampled part sits lower
    z[3, 32768:] = torch.round(z[3, 32768:] * 4) / 4   # ties outside the sample
    for p in (0.5, 0.9, 0.99):
        check_cut(z, 0.7, p, what="unpredicted")
    check_cut(syn.normal((3, 5001), 12, "topp_odd", std=2.0), 0.7, 0.95, what="V % 4 != 0")


def test_cut_largest_vocabulary():
    """Rows of 2^24 - 1 entries, the longest the calls allow (each mass bin's
    64-bit fixed-point sum is still exact there): cut, mask and oracle agree."""
    check_cut(syn.normal((2, (1 << 24) - 1), 13, "topp_huge", std=2.0), 0.7, 0.99, what="V=2^24-1")


def test_cut_full_vocabulary_rows():
    zt, zd = syn.logits_pair(32, 8, 151936, 2.0, 1.0, seed=3)
    rows = zt.reshape(-1, 151936)
    dev = cuda()
    print("[top_p cut] full vocabulary, 256 rows (oracle on 16)", flush=True)
    cut, kept = dfl.dflash_top_p_cut(rows.to(dev), 0.7, 0.99, want_kept=True)
    _, kept_m = dfl.dflash_top_p_mask(rows.to(dev), 0.7, 0.99, want_kept=True)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_m.cpu())
    pick = torch.tensor([0, 17, 40, 63, 77, 90, 111, 128, 130, 151, 170, 191, 200, 223, 240, 255])
    check_cut(rows[pick].contiguous(), 0.7, 0.99, what="full V sample")


def _same(a, b, what):
    assert torch.equal(a.cpu(), b.cpu()), what


@pytest.mark.parametrize("B,G,V,P", [(4, 8, 5000, 0.9), (3, 5, 5000, 1e-6), (32, 8, 151936, 0.99)])
def test_topk_and_verify_with_cuts_equal_masked_rows(B, G, V, P):
    """The cut-aware scans reproduce, bit for bit, the same kernels run on
    rows masked to the same nuclei: top-k, log-normaliser and draws
    (greedy and sampled, k beyond a tiny nucleus), and verification with and
    without the draft normaliser and with deterministic drafts."""
    T = 0.7
    print(f"[top_p cut] consumers B={B} G={G} V={V} top_p={P}", flush=True)
    dev = cuda()
    zt, zd = syn.logits_pair(B, G, V, 2.0, 1.0, seed=5)
    zt, zd = zt.to(dev), zd.to(dev)
    tc, _ = dfl.dflash_top_p_cut(zt, T, P)
    dc, _ = dfl.dflash_top_p_cut(zd, T, P)
    mt, _ = dfl.dflash_top_p_mask(zt, T, P)
    md, _ = dfl.dflash_top_p_mask(zd, T, P)
    seeds = syn.philox_seeds(B, 7).to(dev)
    for temp, k in ((0.0, 8), (T, 8), (T, 64)):
        a = dfl.dflash_topk(zd, k, temp, seeds=seeds, step=2, cut=dc)
        b = dfl.dflash_topk(md, k, temp, seeds=seeds, step=2)
        for key in ("idx", "val", "draft"):
            _same(a[key], b[key], (temp, k, key))
        if temp > 0:
            _same(a["lse"].view(torch.int64), b["lse"].view(torch.int64), (temp, k, "lse"))
    tk = dfl.dflash_topk(md, 4, T, seeds=seeds, step=2)
    for step in range(3):
        for use_lse in (True, False):
            lse = tk["lse"] if use_lse else None
            a = dfl.spec_verify(zt, zd, tk["draft"], T, seeds=seeds, step=step, draft_lse=lse,
                                target_cut=tc, draft_cut=dc)
            b = dfl.spec_verify(mt, md, tk["draft"], T, seeds=seeds, step=step, draft_lse=lse)
            for key in ("accept_len", "out_tokens", "accepted"):
                _same(a[key], b[key], (step, use_lse, key))
        a = dfl.spec_verify(zt, None, tk["draft"], T, seeds=seeds, step=step, target_cut=tc)
        b = dfl.spec_verify(mt, None, tk["draft"], T, seeds=seeds, step=step)
        for key in ("accept_len", "out_tokens", "accepted"):
            _same(a[key], b[key], (step, "deterministic", key))
    torch.cuda.synchronize()


def test_sampling_and_verification_with_cuts_against_the_oracle():
    """Top-p decoding through cuts: the GPU's cuts name the oracle's nuclei;
    the draws and verification through them meet the unmasked bar against
    the oracle run on the oracle's masked rows."""
    from test_gpu_topk_verify import _topk_case, _verify_case
    B, G, V, T, P = 4, 8, 5000, 0.7, 0.9
    zt, zd = syn.logits_pair(B, G, V, 2.0, 1.0, seed=4)
    dev = cuda()
    tc, _ = dfl.dflash_top_p_cut(zt.to(dev), T, P)
    dc, _ = dfl.dflash_top_p_cut(zd.to(dev), T, P)
    torch.cuda.synchronize()
    rt, _ = oracle.top_p_mask(to64(zt), f32(T), f32(P))
    rd, _ = oracle.top_p_mask(to64(zd), f32(T), f32(P))
    for cut, z, ref in ((tc, zt, rt), (dc, zd, rd)):
        lg, ix = (to64(t) for t in dfl.nucleus_cut_values(cut.cpu()))
        z64 = to64(z)
        for b in range(B):
            for g in range(G):
                np.testing.assert_array_equal(np.isfinite(ref[b, g]),
                                              keep_rule(z64[b, g], lg[b, g], ix[b, g]))
    seeds = syn.philox_seeds(B, 3)
    for step in range(3):
        tk = _topk_case(zd, 8, T, seeds, step=step, what=f"cut drafter rows {step}", cut=dc.cpu(),
                        z_ref=rd)
        drafts = to64(tk["draft"])[:, :G - 1]
        assert np.isfinite(np.take_along_axis(rd[:, :G - 1], drafts[..., None], -1)).all()
        for use_lse in (True, False):
            _verify_case(zt, zd, torch.from_numpy(drafts.astype(np.int64)), T, seeds, step=step,
                         use_lse=use_lse, what=f"cut rows {step}", target_cut=tc.cpu(),
                         draft_cut=dc.cpu(), zt_ref=rt, zd_ref=rd)
