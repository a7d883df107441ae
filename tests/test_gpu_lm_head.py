"""GPU parity of dflash_lm_head_topk (LM head with the top-k / normaliser /
draft epilogue) against the fp64 oracle, through the C ABI.

The GPU logits are bf16 products accumulated in fp32; the oracle's are exact
dot products in fp64.  Every logit therefore carries an error bounded by
tol = 2^-24 (d/32 + 32) sum_j |h_j W_vj| (fp32 roundings of the 32-term MFMA
partial sums and of the d/32 accumulations), which the bar propagates:
  * top-k values within tol of the oracle's logit at the same index; indices
    bit-exact wherever the oracle's values at that rank are separated by more
    than 2 tol (elsewhere the GPU's pick must be one of the near-equal ones);
  * lse within 1e-5 + tol / T;
  * greedy drafts equal top-1; sampled drafts (one inverse-CDF draw over the
    whole row at the purpose-0 uniform) bit-exact except where that uniform
    lies within 2 tol / T + 1e-5 of every CDF boundary between the two
    choices.
The temperature is the fp32 value the library receives, widened to fp64.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax
from scipy.stats import chi2

import oracle
import block_drafting_context_amd as dfl
from block_drafting_context_amd import synthetic as syn
from parity_util import cuda, to64

pytestmark = pytest.mark.gpu
U24 = 2.0 ** -24


def f32(x):
    return float(np.float32(x))


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(t):
    return t.double().numpy()


def abs_bound(h, w, rows):
    """sum_j |h_rj W_vj| for the checked rows, exactly (fp64, W in chunks of
    8,192 rows at large sizes)."""
    hb = np.abs(f64(h[rows]))
    out = np.empty((len(rows), w.shape[0]))
    for c in range(0, w.shape[0], 8192):
        out[:, c:c + 8192] = hb @ np.abs(f64(w[c:c + 8192])).T
    return out


def draw_ok(z, T, seed, step, b, g, got, ref, eps):
    """The two draws may differ only where the uniform lies within eps of every
    CDF boundary between them (weights in fp64 by scipy)."""
    if got == ref:
        return True
    w = softmax(z / T)
    if w[got] <= 0:
        return False
    u0 = oracle.uniform(seed, step, b, g, 0)
    c = np.cumsum(w) / w.sum()
    lo, hi = min(got, ref), max(got, ref)
    return bool(np.all(np.abs(c[lo:hi] - u0) < eps))


def run_case(h, w, gamma, k, T, seeds=None, step=0, check_rows=None, what=""):
    rows, d = h.shape
    V = w.shape[0]
    print(f"[lm_head] {what} rows={rows} d={d} V={V} k={k} T={T}", flush=True)
    dev = cuda()
    sd = None if seeds is None else seeds.to(dev)
    res = dfl.dflash_lm_head_topk(h.to(dev), w.to(dev), gamma, k, T, seeds=sd, step=step)
    torch.cuda.synchronize()
    idx, val = to64(res["idx"]), to64(res["val"])
    lse, draft = to64(res["lse"]), to64(res["draft"])
    assert ((idx >= 0) & (idx < V)).all() and np.isfinite(val).all()
    assert ((draft >= 0) & (draft < V)).all()
    for r in range(rows):  # sorted by (value desc, index asc), distinct
        assert len(set(idx[r])) == k
        assert all(val[r, i] > val[r, i + 1] or (val[r, i] == val[r, i + 1] and idx[r, i] < idx[r, i + 1])
                   for i in range(k - 1)), r
    rows_chk = np.arange(rows) if check_rows is None else np.asarray(check_rows)
    Tf = f32(T)
    sd_np = None if seeds is None else to64(seeds).astype(np.uint64)
    ref = oracle.lm_head_topk(bits(h)[rows_chk], bits(w), gamma, k, Tf, seeds=sd_np, step=step,
                              row_id=rows_chk, want_z=True)
    tol_all = U24 * (d / 32 + 32) * abs_bound(h, w, rows_chk)
    for i, r in enumerate(rows_chk):
        z = ref["z"][i]
        tol = tol_all[i]
        gi = idx[r]
        assert np.all(np.abs(val[r] - z[gi]) <= tol[gi]), (r, "values")
        order = ref["idx"][i]
        for q in range(k):
            if gi[q] != order[q]:
                assert abs(z[gi[q]] - z[order[q]]) <= tol[gi[q]] + tol[order[q]], (r, q, gi[q], order[q])
        tmax = float(tol.max())
        if T == 0:
            assert np.isnan(lse[r])
            assert draft[r] == gi[0]
        else:
            assert abs(lse[r] - ref["lse"][i]) <= 1e-5 + tmax / Tf, (r, lse[r], ref["lse"][i])
            b, g = divmod(int(r), gamma)
            assert draw_ok(z, Tf, int(sd_np[b]), step, b, g, int(draft[r]), int(ref["draft"][i]),
                           2 * tmax / Tf + 1e-5), (r, draft[r], ref["draft"][i])
    return res


def test_small_sampled_every_row():
    h, w = syn.lm_head_inputs(24, 256, 1000, seed=1)       # 8 segments, the last one 104 wide
    run_case(h, w, 8, 8, 0.7, seeds=syn.philox_seeds(3, 5), step=3, what="small")


@pytest.mark.parametrize("k", [1, 4, 5, 13, 16])
@pytest.mark.parametrize("T", [0.0, 0.9])
def test_k_and_temperature(k, T):
    h, w = syn.lm_head_inputs(16, 128, 777, seed=2)
    run_case(h, w, 4, k, T, seeds=syn.philox_seeds(4, 1) if T > 0 else None, step=1,
             what=f"k={k}")


def test_equal_logits_take_lower_index_and_overflow_a_slot():
    """Forty identical weight rows in one segment give forty equal maxima (more
    than a segment's candidate slot holds); more ties across segments."""
    h, w = syn.lm_head_inputs(8, 128, 1200, seed=3)
    w = w.clone()
    w[130:170] = w[5] * 4                 # equal and largest: entries 130..169
    w[1000:1003] = w[5] * 4               # the same value in a later segment
    res = run_case(h, w, 8, 16, 0.0, what="ties greedy")
    # rows where the planted value is the maximum: the top 16 are 130..145
    idx = to64(res["idx"])
    z = f64(h) @ f64(w).T
    for r in range(8):
        if np.argmax(z[r]) == 130:
            np.testing.assert_array_equal(idx[r], np.arange(130, 146))
    run_case(h, w, 8, 16, 0.5, seeds=syn.philox_seeds(1, 2), what="ties sampled")


def test_more_equal_maxima_than_the_finalize_ranks_at_once():
    """Four hundred identical weight rows (entries 0..399, four segments) give
    more entries at or above the finalize's threshold than it ranks in one
    step (256), so it selects through its block-wide rounds."""
    h, w = syn.lm_head_inputs(8, 128, 1200, seed=5)
    w = w.clone()
    w[0:400] = (h[0].float() * 0.2).to(w.dtype)  # far above every other logit of row 0
    res = run_case(h, w, 8, 16, 0.0, what="400 ties greedy")
    idx = to64(res["idx"])
    z = f64(h) @ f64(w).T
    hit = 0
    for r in range(8):
        if np.argmax(z[r]) == 0:
            np.testing.assert_array_equal(idx[r], np.arange(16))
            hit += 1
    assert hit > 0
    run_case(h, w, 8, 16, 0.5, seeds=syn.philox_seeds(1, 3), what="400 ties sampled")


def test_more_rows_than_one_pass():
    h, w = syn.lm_head_inputs(300, 64, 513, seed=4)      # two passes over the weights
    run_case(h, w, 6, 8, 1.0, seeds=syn.philox_seeds(50, 9), step=2, what="300 rows")


def test_uneven_segment_runs():
    """547 segments over 256 workgroups: runs of 2 and 3 segments (a 3-segment
    run ends in a half tile), the last segment ragged.  Planted maxima in the
    upper vocabulary and in the ragged segment put top-k entries there."""
    h, w = syn.lm_head_inputs(40, 256, 70000, seed=8)
    w = w.clone()
    w[66000:66006] = w[66000:66006] * 3
    w[69950:69953] = w[69950:69953] * 3        # inside the ragged last segment
    run_case(h, w, 8, 8, 0.7, seeds=syn.philox_seeds(5, 3), step=4,
             check_rows=[0, 7, 20, 39], what="uneven runs")
    run_case(h, w, 8, 16, 0.0, check_rows=[1, 38], what="uneven runs greedy")


def test_long_segment_runs():
    """911 segments over 256 workgroups: runs of 3 and 4 segments."""
    h, w = syn.lm_head_inputs(16, 128, 116600, seed=9)
    run_case(h, w, 8, 8, 0.9, seeds=syn.philox_seeds(2, 4), check_rows=[0, 9, 15],
             what="long runs")


def test_uneven_runs_over_two_passes():
    """300 rows (two passes over the weights) with uneven segment runs."""
    h, w = syn.lm_head_inputs(300, 128, 70000, seed=10)
    run_case(h, w, 6, 8, 1.0, seeds=syn.philox_seeds(50, 1), step=1,
             check_rows=[0, 1, 255, 256, 299], what="uneven runs, 300 rows")


@pytest.mark.parametrize("V,T", [(4, 0.0), (4, 0.9), (5, 0.9)])
def test_vocabulary_as_small_as_k(V, T):
    """The smallest vocabularies the call allows: V = k (every entry is a
    candidate) and V = k + 1, in one partial segment."""
    h, w = syn.lm_head_inputs(6, 64, V, seed=11)
    run_case(h, w, 3, 4, T, seeds=syn.philox_seeds(2, 4) if T > 0 else None, what=f"V={V}")


def test_largest_vocabulary():
    """V = 1,048,576 entries (8,192 segments per row), the largest the call allows."""
    h, w = syn.lm_head_inputs(8, 64, 1 << 20, seed=12)
    run_case(h, w, 8, 16, 0.7, seeds=syn.philox_seeds(1, 5), check_rows=[0, 3, 7], what="V=2^20")


def test_largest_model_width():
    """d_model = 65,536, the largest the call allows: 1,024 K stages per tile."""
    h, w = syn.lm_head_inputs(5, 65536, 600, seed=13)
    run_case(h, w, 5, 8, 0.9, seeds=syn.philox_seeds(1, 6), what="d=65536")


def test_few_rows():
    h, w = syn.lm_head_inputs(8, 512, 4096, seed=5)
    run_case(h, w, 8, 8, 0.7, seeds=syn.philox_seeds(1, 0), what="8 rows")


def test_full_size_sampled_rows():
    """256 drafter rows (32 sequences x 8) over the 151,936-entry vocabulary with
    d_model 5,120: the launch the benchmark times; the oracle checks a sample."""
    h, w = syn.lm_head_inputs(256, 5120, 151936, seed=6)
    run_case(h, w, 8, 8, 0.7, seeds=syn.philox_seeds(32, 0), step=1,
             check_rows=[0, 1, 7, 8, 37, 63, 64, 100, 128, 129, 191, 192, 201, 230, 254, 255],
             what="full size")


def test_draws_follow_softmax():
    """Identical rows with distinct counters: the GPU's draws follow
    softmax(z/T) over 600 entries (chi-square), independent of the oracle."""
    n, V, T = 16384, 600, 1.0
    h1, w = syn.lm_head_inputs(1, 64, V, seed=7, logit_std=1.2)
    h = h1.repeat(n, 1).contiguous()
    print(f"[lm_head] chi-square rows={n} V={V}", flush=True)
    dev = cuda()
    res = dfl.dflash_lm_head_topk(h.to(dev), w.to(dev), 1, 1, T,
                                  seeds=torch.full((n,), 11, dtype=torch.int64, device=dev))
    torch.cuda.synchronize()
    draft = to64(res["draft"])
    p = softmax((f64(h1) @ f64(w).T)[0] / T)
    counts = np.bincount(draft, minlength=V)
    ex = p * n
    small = ex < 5
    obs = np.append(counts[~small], counts[small].sum())
    exp_ = np.append(ex[~small], ex[small].sum())
    stat = ((obs - exp_) ** 2 / exp_).sum()
    assert stat < chi2.ppf(1 - 1e-6, len(obs) - 1), stat
