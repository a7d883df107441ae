"""GPU parity of dflash_context_fuse against the fp64 oracle (C ABI).

Bar (H_t and the appended K/V rows): max|err| <= 1e-2 * max|ref| + 1e-3, the
attention bar, since both come from bf16 products with fp32 accumulation (and
the GPU rounds H_t to bf16 before the K/V projection).  Slots no row addresses
must be left bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import block_drafting_context_amd as dfl
from block_drafting_context_amd import synthetic as syn
from parity_util import ATTN_ABS, ATTN_REL, assert_close_scaled, cuda, to64

pytestmark = pytest.mark.gpu


def _case(rows, n_taps, d_tgt, d_model, NL, NKV, DH, W, B, row_seq, row_pos, seed, sample=None,
          gain_random=True):
    print(f"[fuse] rows={rows} kx={n_taps * d_tgt} d_model={d_model} kv={NL * 2 * NKV * DH} "
          f"B={B} W={W}", flush=True)
    dev = cuda()
    t = syn.fuse_inputs(rows, n_taps, d_tgt, d_model, NL, NKV, DH, seed, device=dev,
                        gain_random=gain_random)
    ring = syn.normal((NL, 2, B, NKV, W, DH), seed, "ring", dtype=torch.bfloat16, device=dev)
    ring0 = ring.clone()
    rs = torch.as_tensor(row_seq, dtype=torch.int32, device=dev)
    rp = torch.as_tensor(row_pos, dtype=torch.int64, device=dev)
    h = torch.empty((rows, d_model), dtype=torch.bfloat16, device=dev)
    dfl.dflash_context_fuse(t["x"], t["w_c"], t["gain"], 1e-6, t["w_kv"], rs, rp, ring, n_taps,
                            h_t_out=h)
    torch.cuda.synchronize()
    idx = np.arange(rows) if sample is None else np.asarray(sample)
    # oracle on the sampled rows, each written to its own slot 0 of a compact ring
    x = to64(t["x"])[idx]
    href, kv = oracle.context_fuse(x, to64(t["w_c"]), to64(t["gain"]), float(np.float32(1e-6)),
                                   to64(t["w_kv"]), np.arange(len(idx)), np.zeros(len(idx)),
                                   np.zeros((NL, 2, len(idx), NKV, 1, DH)), NL, NKV, DH)
    assert_close_scaled(to64(h)[idx], href, ATTN_REL, ATTN_ABS, "H_t")
    rs_np, rp_np = np.asarray(row_seq), np.asarray(row_pos)
    got = np.stack([to64(ring[:, :, rs_np[r], :, rp_np[r] % W, :]) for r in idx], axis=2)
    assert_close_scaled(got, kv[:, :, :, :, 0, :], ATTN_REL, ATTN_ABS, "K/V rows")
    # untouched slots are bit-identical
    untouched = torch.ones((B, W), dtype=torch.bool, device=dev)
    untouched[rs.long(), rp % W] = False
    changed = (ring.view(torch.int16) != ring0.view(torch.int16))
    changed = changed.any(dim=5).any(dim=3).any(dim=1).any(dim=0)  # [B, W]
    assert not bool((changed & untouched).any())


def test_fuse_small_ragged_rows():
    rows, B, W = 40, 3, 64
    rng = np.random.default_rng(0)
    seqs = rng.integers(0, B, rows)
    pos = np.zeros(rows, dtype=np.int64)
    nxt = {s: int(rng.integers(0, 500)) for s in range(B)}
    for r in range(rows):
        pos[r] = nxt[seqs[r]]
        nxt[seqs[r]] += 1
    _case(rows, 5, 128, 256, 2, 2, 64, W, B, seqs, pos, seed=1)


def test_fuse_partial_second_row_tile():
    """300 rows: two 256-row tiles of the GEMMs, the second one partial (its
    missing rows read a valid row and are never stored), including the K/V
    projection's reads of H_t in K slabs; every row against the oracle."""
    rows, B, W = 300, 5, 128
    seqs = np.arange(rows) % B
    pos = np.arange(rows) // B + 7
    _case(rows, 5, 128, 256, 2, 2, 64, W, B, seqs, pos, seed=5)


@pytest.mark.parametrize("rows,n_taps,d_tgt,d_model,NL,NKV,DH,W,B", [
    (1, 5, 64, 128, 1, 2, 32, 64, 1),       # one row, the smallest d_model, d_head 32
    (17, 3, 192, 384, 1, 2, 96, 128, 4),    # three taps, d_model 384 (a ragged 160-column tile), d_head 96
    (9, 1, 256, 8192, 1, 1, 64, 64, 3),     # one tap, the largest d_model
])
def test_fuse_shape_edges(rows, n_taps, d_tgt, d_model, NL, NKV, DH, W, B):
    # distinct (sequence, slot) targets, positions past the window on some rows
    seqs = np.arange(rows) % B
    pos = (np.arange(rows) // B) * 7 + 3 * W // 2
    _case(rows, n_taps, d_tgt, d_model, NL, NKV, DH, W, B, seqs, pos, seed=6 + rows)


def test_fuse_wraps_ring():
    """Positions 36..99 of one sequence in a 64-slot ring: every slot is written
    once and the row at position p lands in slot p mod 64."""
    pos = np.arange(36, 100)
    _case(len(pos), 5, 64, 128, 1, 1, 64, 64, 1, np.zeros(len(pos), int), pos, seed=2)


def test_fuse_full_drafter_step_sampled_rows():
    """Batch 64 x 8 new tokens: [512 x 25600] x [25600 x 5120], RMSNorm, then
    5 layers x K/V x 8 heads x 128 appended to 4,096-slot rings (16 sampled rows
    checked against the oracle, all untouched slots checked bit-exact)."""
    B, W, per = 64, 4096, 8
    rows = B * per
    seqs = np.repeat(np.arange(B), per)
    pos = np.tile(np.arange(per), B) + (W + 8 - per)
    sample = np.random.default_rng(3).choice(rows, 16, replace=False)
    _case(rows, 5, 5120, 5120, 5, 8, 128, W, B, seqs, pos, seed=3, sample=sample,
          gain_random=False)


def test_fuse_serving_step_sampled_rows():
    """The throughput workload's fusion: 32 sequences x 8 newly verified tokens
    (256 rows, the launch configuration the bench times), positions ctx_len - 8
    .. ctx_len - 1 of context lengths uniform in [512, 131072], so the rows land
    at wrapped slots of the 4,096-slot rings (16 sampled rows against the oracle,
    all untouched slots bit-exact)."""
    B, W, per = 32, 4096, 8
    rows = B * per
    cl = syn.ctx_lengths(B, 512, 131072, 3).numpy().astype(np.int64)
    seqs = np.repeat(np.arange(B), per)
    pos = np.repeat(cl, per) - per + np.tile(np.arange(per), B)
    sample = np.random.default_rng(4).choice(rows, 16, replace=False)
    _case(rows, 5, 5120, 5120, 5, 8, 128, W, B, seqs, pos, seed=4, sample=sample,
          gain_random=False)
