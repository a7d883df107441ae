"""Pins for the oracle's context fusion and the position weights (CPU only).

Context fusion follows "DFlash vs DFlash 2", "Conditioning on the target
model": H_t = RMSNorm(W_c [H^(l1); ...; H^(l5)]) and the context half of each
draft layer's K_i = W_i^K H_t, V_i = W_i^V H_t.  Pins: numpy matmul (library)
for both products, RMSNorm closed forms (constant row, unit mean square, scale
invariance, direction), and the ring-append invariant.  Position weights follow
"Training with anchors", equation for w_k; pinned by tests/golden values and
closed forms.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_drafting_context_amd import synthetic as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fuse_case(rows=6, n_taps=5, d_tgt=16, d_model=32, NL=2, NKV=2, DH=8, W=16, B=3, seed=0,
               gain_random=True):
    t = syn.fuse_inputs(rows, n_taps, d_tgt, d_model, NL, NKV, DH, seed, dtype=torch.float32,
                        gain_random=gain_random)
    x, wc, wkv, g = (t[k].double().numpy() for k in ("x", "w_c", "w_kv", "gain"))
    rng = np.random.default_rng(seed)
    ring = rng.standard_normal((NL, 2, B, NKV, W, DH))
    return x, wc, wkv, g, ring


def test_projections_match_numpy_matmul():
    x, wc, wkv, g, ring = _fuse_case()
    NL, _, B, NKV, W, DH = ring.shape
    row_seq = np.array([0, 2, 2, 1, 0, 2])
    row_pos = np.array([3, 16, 40, 0, 36, 17])  # no two rows share (sequence, slot)
    h, new = oracle.context_fuse(x, wc, g, 1e-6, wkv, row_seq, row_pos, ring, NL, NKV, DH)
    y = x @ wc.T
    # direction of each H_t row is that of g * y (RMSNorm only rescales per row)
    for r in range(6):
        ref = g * y[r]
        cos = h[r] @ ref / (np.linalg.norm(h[r]) * np.linalg.norm(ref))
        assert abs(cos - 1.0) < 1e-12
    kv = h @ wkv.T
    for r in range(6):
        for c in range(kv.shape[1]):
            d, hh = c % DH, (c // DH) % NKV
            kvi, layer = (c // (DH * NKV)) % 2, c // (DH * NKV * 2)
            assert abs(new[layer, kvi, row_seq[r], hh, row_pos[r] % W, d] - kv[r, c]) < 1e-12


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    x, wc, wkv, g, ring = _fuse_case(gain_random=False)
    NL, _, B, NKV, W, DH = ring.shape
    rs, rp = np.zeros(6, int), np.arange(6)
    h, _ = oracle.context_fuse(x, wc, g, 0.0, wkv, rs, rp, ring, NL, NKV, DH)
    np.testing.assert_allclose((h ** 2).mean(1), 1.0, atol=1e-13)
    h2, _ = oracle.context_fuse(37.5 * x, wc, g, 0.0, wkv, rs, rp, ring, NL, NKV, DH)
    np.testing.assert_allclose(h2, h, atol=1e-12)


def test_rmsnorm_constant_row_closed_form():
    """All rows of W_c equal => every output feature equals c; RMSNorm gives
    c / sqrt(c^2 + eps) * g."""
    x, wc, wkv, g, ring = _fuse_case()
    NL, _, B, NKV, W, DH = ring.shape
    wc[:] = wc[0]
    eps = 0.05
    h, _ = oracle.context_fuse(x, wc, g, eps, wkv, np.zeros(6, int), np.arange(6), ring, NL, NKV,
                               DH)
    c = x @ wc[0]
    np.testing.assert_allclose(h, (c / np.sqrt(c * c + eps))[:, None] * g[None, :], atol=1e-13)


@pytest.mark.parametrize("p0,n", [(0, 5), (14, 5), (3, 16), (30, 40)])
def test_ring_append_equals_last_window_of_history(p0, n):
    """Appending positions [p0, p0+n) of one sequence (after a history [0, p0))
    leaves the ring equal to the last min(p0+n, W) rows of the linear history;
    other sequences' rows are untouched."""
    rows, W = p0 + n, 16
    x, wc, wkv, g, ring = _fuse_case(rows=rows, W=W, seed=p0 + n)
    NL, _, B, NKV, _, DH = ring.shape
    all_h, _ = oracle.context_fuse(x, wc, g, 1e-6, wkv, np.ones(rows, int), np.arange(rows), ring,
                                   NL, NKV, DH)
    hist = all_h @ wkv.T  # [rows, NL*2*NKV*DH] linear history of every layer's K/V
    _, r1 = oracle.context_fuse(x[:p0], wc, g, 1e-6, wkv, np.ones(p0, int), np.arange(p0), ring,
                                NL, NKV, DH) if p0 else (None, ring.copy())
    _, r2 = oracle.context_fuse(x[p0:], wc, g, 1e-6, wkv, np.ones(n, int), np.arange(p0, rows),
                                r1, NL, NKV, DH)
    hist = hist.reshape(rows, NL, 2, NKV, DH)
    for pos in range(max(0, rows - W), rows):
        np.testing.assert_allclose(r2[:, :, 1, :, pos % W, :], hist[pos], atol=1e-12)
    np.testing.assert_array_equal(r2[:, :, 0], ring[:, :, 0])
    np.testing.assert_array_equal(r2[:, :, 2], ring[:, :, 2])
    if rows < W:
        np.testing.assert_array_equal(r2[:, :, 1, :, rows:], ring[:, :, 1, :, rows:])


def test_position_weights_golden_and_closed_forms():
    table = {}
    with open(os.path.join(GOLDEN, "position_weights.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                g, k, w = line.split()
                table[(int(g), int(k))] = float(w)
    for gamma in (8, 16):
        w = oracle.position_weights(gamma)
        assert w[0] == 1.0
        ratios = w[1:] / w[:-1]
        np.testing.assert_allclose(ratios, ratios[0], rtol=1e-14)
        assert abs(ratios[0] ** gamma - 1 / math.e) < 1e-14
        assert abs(w[gamma // 2] - 1 / math.sqrt(math.e)) < 1e-15
        for (gg, k), v in table.items():
            if gg == gamma:
                assert abs(w[k - 1] - v) < 5e-7
