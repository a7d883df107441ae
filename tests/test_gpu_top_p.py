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
    pick = torch.tensor([0, 77, 130, 255])
    print("[top_p] full vocabulary, 256 rows (oracle on 4)", flush=True)
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
