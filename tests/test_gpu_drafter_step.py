"""The full drafter step at batch 64, end to end on the GPU, against the fp64
oracle chain (C ABI): context fusion of the 8 newly verified tokens of each of
64 sequences (512 rows: [512 x 25,600] . [25,600 x 5,120], RMSNorm, K/V of 5
layers x 8 heads x 128 appended to the 4,096-slot rings), then 5 stacked
block-attention layers (40q / 8kv x 128) reading the rings just written, then
top-8 + drafted tokens and sampled verification at T = 0.7 over 151,936
entries.  "Beam 1.0 DFlash2", "Model" (5 drafter layers, taps, heads);
"DFlash vs DFlash 2", "Conditioning on the target model" (H_t, K_i, V_i) and
"The problem: one expensive token at a time" (verification).

The oracle fuses the checked sequences' rows itself and attends over its own
fp64 K/V rows (the other ring slots are the same seeded input on both sides),
so fusion errors propagate into the attention comparison.  Bars: fusion and
attention max|err| <= 1e-2 max|ref| + 1e-3; top-k exact; draws and accept
decisions exact except at the documented uniform boundaries.  Context
lengths are mixed and include the extremes: 8 (the ring holds only the new
rows), 4,095, 4,096, 4,104 and 131,072.
"""
import numpy as np
import pytest
import torch

import oracle
import block_drafting_context_amd as dfl
from block_drafting_context_amd import synthetic as syn
from parity_util import (ATTN_ABS, ATTN_REL, U_EXEMPT, assert_close_scaled, cuda,
                         draw_boundary_ok, to64)

pytestmark = pytest.mark.gpu

B, G, W, NL, NKV, HQ, DH, TAPS, DT, DM, V, K = 64, 8, 4096, 5, 8, 40, 128, 5, 5120, 5120, 151936, 8
T = float(np.float32(0.7))
SEED = 5


def test_full_drafter_step_batch64_end_to_end():
    dev = cuda()
    print("[step64] inputs", flush=True)
    cl = syn.ctx_lengths(B, 8, 131072, SEED).numpy().astype(np.int64)
    cl[:5] = [8, 4095, 4096, 4104, 131072]
    chk = np.array([0, 1, 2, 3, 4, 17, 40, 63])
    f = syn.fuse_inputs(B * G, TAPS, DT, DM, NL, NKV, DH, SEED, device=dev)
    ring = syn.normal((NL, 2, B, NKV, W, DH), SEED, "ring", dtype=torch.bfloat16, device=dev)
    ring0 = ring[:, :, torch.as_tensor(chk, device=dev)].cpu()       # the checked sequences' input
    seqs = np.repeat(np.arange(B), G)
    pos = np.repeat(cl, G) - G + np.tile(np.arange(G), B)
    h = torch.empty((B * G, DM), dtype=torch.bfloat16, device=dev)
    ctx = torch.as_tensor(cl, device=dev)

    print("[step64] fuse + 5 attention layers + top-k + verify", flush=True)
    dfl.dflash_context_fuse(f["x"], f["w_c"], f["gain"], 1e-6, f["w_kv"],
                            torch.as_tensor(seqs, dtype=torch.int32, device=dev),
                            torch.as_tensor(pos, device=dev), ring, TAPS, h_t_out=h)
    att_in, att_out = [], []
    for i in range(NL):
        q = syn.normal((B, G, HQ, DH), SEED, f"q{i}", std=3.0, dtype=torch.bfloat16, device=dev)
        kb = syn.normal((B, G, NKV, DH), SEED, f"k_blk{i}", dtype=torch.bfloat16, device=dev)
        vb = syn.normal((B, G, NKV, DH), SEED, f"v_blk{i}", dtype=torch.bfloat16, device=dev)
        att_out.append(dfl.dflash_block_attn(q, kb, vb, ring[i, 0], ring[i, 1], ctx,
                                             1 / np.sqrt(DH)))
        att_in.append((q, kb, vb))
    zt, zd = syn.logits_pair(B, G, V, 3.0, 1.5, SEED, device=dev)
    seeds = syn.philox_seeds(B, 0, device=dev)
    tk = dfl.dflash_topk(zd, K, T, seeds=seeds, step=2)
    vr = dfl.spec_verify(zt, zd, tk["draft"], T, seeds=seeds, step=2, draft_lse=tk["lse"])
    torch.cuda.synchronize()

    print("[step64] oracle: fusion of the checked sequences' rows", flush=True)
    rows = (chk[:, None] * G + np.arange(G)[None, :]).reshape(-1)
    href, kv = oracle.context_fuse(to64(f["x"])[rows], to64(f["w_c"]), to64(f["gain"]),
                                   float(np.float32(1e-6)), to64(f["w_kv"]),
                                   np.repeat(np.arange(len(chk)), G), np.tile(np.arange(G), len(chk)),
                                   np.zeros((NL, 2, len(chk), NKV, G, DH)), NL, NKV, DH)
    assert_close_scaled(to64(h)[rows], href, ATTN_REL, ATTN_ABS, "H_t")
    slots = (cl[chk][:, None] - G + np.arange(G)[None, :]) % W          # [n_chk, G]
    got_kv = np.stack([to64(ring[:, :, int(s)][:, :, :, torch.as_tensor(slots[c], device=dev)])
                       for c, s in enumerate(chk)], axis=2)             # [NL,2,n_chk,NKV,G,DH]
    assert_close_scaled(got_kv, kv, ATTN_REL, ATTN_ABS, "K/V rows")

    print("[step64] oracle: 5 attention layers on the checked sequences", flush=True)
    for i in range(NL):
        rk = to64(ring0[i, 0])
        rv = to64(ring0[i, 1])
        for c in range(len(chk)):
            rk[c][:, slots[c], :] = kv[i, 0, c]
            rv[c][:, slots[c], :] = kv[i, 1, c]
        q, kb, vb = (to64(t[torch.as_tensor(chk, device=dev)]) for t in att_in[i])
        ref = oracle.block_attn(q, kb, vb, rk, rv, cl[chk], 1 / np.sqrt(DH))
        assert_close_scaled(to64(att_out[i])[chk], ref, ATTN_REL, ATTN_ABS, f"attention layer {i}")

    print("[step64] oracle: top-k, draws and verification of all 64 sequences", flush=True)
    sd = np.arange(B, dtype=np.uint64)
    z_t, z_d = to64(zt), to64(zd)
    ref_tk = oracle.draft_rows(z_d, K, T, seeds=sd, step=2)
    np.testing.assert_array_equal(to64(tk["idx"]), ref_tk["idx"])
    assert np.abs(to64(tk["lse"]) - ref_tk["lse"]).max() < 1e-6
    drafts = to64(tk["draft"])
    same = np.ones(B, dtype=bool)
    for b in range(B):
        for g in range(G):
            if drafts[b, g] != ref_tk["draft"][b, g]:
                u = oracle.uniform(b, 2, b, g, 0)
                assert draw_boundary_ok(z_d[b, g], T, u, int(drafts[b, g]),
                                        int(ref_tk["draft"][b, g])), (b, g)
                same[b] = False
    ref_v = oracle.spec_verify(z_t, z_d, ref_tk["draft"][:, :G - 1], T, seeds=sd, step=2)
    j, out, acc = to64(vr["accept_len"]), to64(vr["out_tokens"]), to64(vr["accepted"])
    checked = 0
    for b in np.nonzero(same)[0]:
        if np.any(acc[b] != ref_v["accepted"][b]):
            for r in np.nonzero(acc[b] != ref_v["accepted"][b])[0]:
                u = oracle.uniform(int(b), 2, int(b), int(r), 1)
                assert abs(u - min(1.0, ref_v["ratio"][b, r])) < U_EXEMPT, (b, r)
            continue
        assert j[b] == ref_v["accept_len"][b], b
        jj = int(j[b])
        np.testing.assert_array_equal(out[b, :jj], ref_v["out_tokens"][b, :jj])
        np.testing.assert_array_equal(out[b, jj + 1:], ref_v["out_tokens"][b, jj + 1:])
        if out[b, jj] != ref_v["out_tokens"][b, jj]:
            u = oracle.uniform(int(b), 2, int(b), jj, 2)
            assert draw_boundary_ok(z_t[b, jj], T, u, int(out[b, jj]), int(ref_v["out_tokens"][b, jj]),
                                    residual_q=z_d[b, jj] if jj < G - 1 else None), b
        checked += 1
    assert checked >= B - 2
