"""The library built with device checks (libdflash_checked.so) through the C ABI.

Valid device data records no violation; each violated device-data
precondition sets its DFLASH_VIOLATION_* bit in the GPU's word (token ids
outside the vocabulary, negative context lengths, fused rows with an invalid
sequence or position, two fused rows on one ring slot); and the checked build
computes what the release build computes on the same inputs (both clamp or
skip a violating value, so every access stays in its buffer; only the
duplicate-slot case leaves the shared slot to whichever write lands last).
"""
import contextlib

import numpy as np
import pytest
import torch

import block_drafting_context_amd as dfl
from block_drafting_context_amd import synthetic as syn
from parity_util import cuda

pytestmark = pytest.mark.gpu
TOKEN, CTX_LEN, ROW, SLOT = 1, 2, 4, 8


@contextlib.contextmanager
def checked_library():
    saved = (dfl._lib, dfl.lib_path)
    dfl._lib, dfl.lib_path = None, dfl.checked_lib_path
    try:
        dfl.load()
        assert dfl.dflash_device_checks() == 1
        yield
    finally:
        dfl._lib, dfl.lib_path = saved


def both(fn, what):
    """fn() with the release library, then with the checked one; returns the
    two results and the violation word the checked run left."""
    print(f"[device checks] {what}", flush=True)
    assert dfl.dflash_device_checks() == 0
    rel = fn()
    torch.cuda.synchronize()
    with checked_library():
        dfl.dflash_violations(clear=True)
        chk = fn()
        torch.cuda.synchronize()
        word = dfl.dflash_violations(clear=True)
    return rel, chk, word


def same(a, b):
    assert torch.equal(a.cpu(), b.cpu())


@pytest.mark.parametrize("ctx,bits", [([256, 17, 0], 0), ([256, -5, 40], CTX_LEN)])
@pytest.mark.parametrize("dtype", [dfl.DTYPE_BF16, dfl.DTYPE_FP32])
def test_attention_context_length(ctx, bits, dtype):
    dev = cuda()
    tdt = torch.bfloat16 if dtype == dfl.DTYPE_BF16 else torch.float32
    a = syn.attention_inputs(3, 8, 40, 8, 128, 256, [max(c, 0) for c in ctx], seed=4, dtype=tdt,
                             device=dev)
    a["ctx_len"] = torch.as_tensor(ctx, dtype=torch.int64, device=dev)

    def run():
        return dfl.dflash_block_attn(a["q"], a["k_blk"], a["v_blk"], a["k_ring"], a["v_ring"],
                                     a["ctx_len"], 1 / np.sqrt(128))
    rel, chk, word = both(run, f"attention ctx={ctx} dtype={dtype}")
    same(rel, chk)
    assert word == bits


@pytest.mark.parametrize("case", ["valid", "sequence", "position", "duplicate"])
def test_fuse_rows_and_slots(case):
    dev = cuda()
    rows, B, W = 8, 4, 64
    f = syn.fuse_inputs(rows, 5, 64, 128, 1, 1, 64, 6, device=dev)
    seq = [0, 0, 1, 1, 2, 2, 3, 3]
    pos = [10, 11, 70, 71, 0, 63, 127, 5]
    if case == "sequence":
        seq[3] = B                 # no such sequence: the row is skipped
    elif case == "position":
        pos[5] = -1                # the row is skipped
    elif case == "duplicate":
        pos[1] = 10 + W            # slot 10 of sequence 0 again
    ring0 = syn.normal((1, 2, B, 1, W, 64), 6, "ring", dtype=torch.bfloat16, device=dev)
    rs = torch.as_tensor(seq, dtype=torch.int32, device=dev)
    rp = torch.as_tensor(pos, dtype=torch.int64, device=dev)

    def run():
        ring = ring0.clone()
        h = torch.empty((rows, 128), dtype=torch.bfloat16, device=dev)
        dfl.dflash_context_fuse(f["x"], f["w_c"], f["gain"], 1e-6, f["w_kv"], rs, rp, ring, 5,
                                h_t_out=h)
        return ring, h
    (rel, hr), (chk, hc), word = both(run, f"fuse {case}")
    same(hr, hc)
    if case == "duplicate":
        keep = torch.ones_like(rel, dtype=torch.bool)
        keep[:, :, 0, :, 10] = False           # the contested slot: either write may land last
        same(rel[keep], chk[keep])
    else:
        same(rel, chk)
    assert word == {"valid": 0, "sequence": ROW, "position": ROW, "duplicate": SLOT}[case]


@pytest.mark.parametrize("T", [0.0, 0.8])
@pytest.mark.parametrize("bad", [False, True])
def test_verify_draft_ids(T, bad):
    dev = cuda()
    B, G, V = 3, 8, 1000
    zt, zd = syn.logits_pair(B, G, V, 2.0, 1.0, seed=7)
    zt, zd = zt.to(dev), zd.to(dev)
    seeds = syn.philox_seeds(B, 2).to(dev) if T > 0 else None
    drafts = dfl.dflash_topk(zd, 4, T, seeds=seeds, step=1)["draft"].clone()
    if bad:
        drafts[0, 2] = V           # past the vocabulary
        drafts[2, 0] = -3

    def run():
        return dfl.spec_verify(zt, zd if T > 0 else None, drafts, T, seeds=seeds, step=1)
    rel, chk, word = both(run, f"verify T={T} bad={bad}")
    for key in ("accept_len", "out_tokens", "accepted"):
        same(rel[key], chk[key])
    assert word == (TOKEN if bad else 0)


@pytest.mark.parametrize("bad", ["none", "candidate", "anchor"])
def test_selector_token_ids(bad):
    dev = cuda()
    B, G, k, V, r = 2, 8, 4, 500, 64
    cand = syn.uniform_int((B, G, k), 0, V - 1, 8, "cand").to(torch.int32).to(dev)
    U = syn.normal((B, G, k), 8, "U", device=dev)
    ea = syn.normal((V, r), 8, "emb_a", std=0.125, dtype=torch.bfloat16, device=dev)
    eb = syn.normal((V, r), 8, "emb_b", std=0.125, dtype=torch.bfloat16, device=dev)
    gate = syn.normal((B, G, r), 8, "gate", dtype=torch.bfloat16, device=dev)
    anchor = torch.tensor([3, 400], dtype=torch.int32, device=dev)
    if bad == "candidate":
        cand[1, 5, 2] = V + 7
    elif bad == "anchor":
        anchor[0] = -1

    def run():
        out = dfl.dflash_select_path(cand, U, ea, eb, gate, anchor)
        return out["path"], out["score"]
    (pr, sr), (pc, sc), word = both(run, f"selector {bad}")
    same(pr, pc)
    same(sr, sc)
    assert word == (0 if bad == "none" else TOKEN)
