"""GPU parity of the candidate selector (dflash_select_path) and of verification
with deterministic drafts (spec_verify with no draft logits), against the oracle.

Selector bar: the path is bit-exact and the path scores equal the oracle's fp64
scores rounded to fp32 (both sides sum the exact bf16 triple products in the
same order in fp64).  Verify bar: as for sampled verification -- accept flags
exact except where the oracle's u is within 1e-6 of p(d), draws exact except
within 1e-6 of a CDF boundary of the residual (p without the rejected draft).
Inputs are seeded and synthetic (block_drafting_context_amd.synthetic)."""
import numpy as np
import pytest
import torch

import block_drafting_context_amd as dfl
import oracle
from block_drafting_context_amd import synthetic as syn
from parity_util import U_EXEMPT, cuda, draw_boundary_ok, to64


def f32(x):
    return float(np.float32(x))


def _inputs(B, G, k, V, r, seed):
    zt, zd = syn.logits_pair(B, G, V, 2.0, 1.0, seed)
    ref = oracle.draft_rows(to64(zd), k, 0.0)
    cand = torch.from_numpy(ref["idx"].astype(np.int32))
    U = torch.from_numpy(ref["val"].astype(np.float32))
    std = 1.0 / np.sqrt(r)
    ea = syn.normal((V, r), seed, "emb_a", std=std, dtype=torch.bfloat16)
    eb = syn.normal((V, r), seed, "emb_b", std=std, dtype=torch.bfloat16)
    gate = syn.normal((B, G, r), seed, "gate", std=1.0, dtype=torch.bfloat16)
    anchor = syn.uniform_int((B,), 0, V - 1, seed, "anchor").to(torch.int32)
    return dict(zt=zt, zd=zd, cand=cand, U=U, ea=ea, eb=eb, gate=gate, anchor=anchor)


def _select_gpu(a):
    dev = cuda()
    out = dfl.dflash_select_path(a["cand"].to(dev), a["U"].to(dev), a["ea"].to(dev),
                                 a["eb"].to(dev), a["gate"].to(dev), a["anchor"].to(dev))
    torch.cuda.synchronize()
    return to64(out["path"]), out["score"].cpu().numpy()


def _select_ref(a):
    return oracle.select_path(to64(a["cand"]), to64(a["U"]), to64(a["ea"]), to64(a["eb"]),
                              to64(a["gate"]), to64(a["anchor"]))


def _check_select(a, what):
    print(f"[select] {what} cand{tuple(a['cand'].shape)} r={a['ea'].shape[1]}", flush=True)
    path, score = _select_gpu(a)
    ref = _select_ref(a)
    np.testing.assert_array_equal(path, ref["path"])
    np.testing.assert_array_equal(score, ref["score"].astype(np.float32))
    return path


@pytest.mark.gpu
def test_select_path_serving_shape():
    """B = 32 sequences, blocks of 8, top-16 over the full vocabulary, r = 64."""
    _check_select(_inputs(32, 8, 16, 151936, 64, seed=21), "serving")


@pytest.mark.gpu
@pytest.mark.parametrize("k,G,r", [(64, 8, 32), (40, 20, 16), (1, 5, 8), (16, 1, 64)])
def test_select_path_chunked_tables_and_edges(k, G, r):
    """k = 64 and k = 40 need several LDS table chunks (the walk crosses chunk
    boundaries); k = 1 and a block of one position are the degenerate walks."""
    _check_select(_inputs(3, G, k, 5000, r, seed=22 + k), f"k={k} G={G}")


@pytest.mark.gpu
@pytest.mark.parametrize("B,G,k,V,r", [(2, 40, 8, 3000, 4096), (2, 4096, 4, 1000, 8)])
def test_select_path_largest_rank_and_block(B, G, k, V, r):
    """The call's limits: embedding rank r = 4,096, and a walk of 4,096 positions."""
    _check_select(_inputs(B, G, k, V, r, seed=31 + r), f"r={r} G={G}")


@pytest.mark.gpu
def test_select_path_planted_chain():
    G, V, r, k = 8, 64, 16, 5
    rng = np.random.default_rng(5)
    chain = rng.permutation(V)[:G + 1]
    ea = np.zeros((V, r))
    eb = np.zeros((V, r))
    gate = np.zeros((1, G, r))
    for t in range(G):
        ea[chain[t], t] = 1.0
        eb[chain[t + 1], t] = 32.0
        gate[0, t, t] = 1.0
    others = [v for v in range(V) if v not in set(chain.tolist())]
    cand = np.zeros((1, G, k), dtype=np.int32)
    U = np.zeros((1, G, k), dtype=np.float32)
    for t in range(G):
        cand[0, t] = [others[(t * 7 + j) % len(others)] for j in range(k - 1)] + [chain[t + 1]]
        U[0, t] = np.linspace(3.0, 1.0, k)
    a = dict(cand=torch.from_numpy(cand), U=torch.from_numpy(U),
             ea=torch.from_numpy(ea).to(torch.bfloat16), eb=torch.from_numpy(eb).to(torch.bfloat16),
             gate=torch.from_numpy(gate).to(torch.bfloat16),
             anchor=torch.tensor([chain[0]], dtype=torch.int32))
    path = _check_select(a, "planted chain")
    assert path[0].tolist() == chain[1:].tolist()


@pytest.mark.gpu
def test_select_path_ties_take_the_first_listed():
    B, G, k, V, r = 2, 3, 8, 100, 8
    cand = torch.from_numpy(np.stack([np.stack([np.random.default_rng(b * 10 + t).permutation(V)[:k]
                                                for t in range(G)]) for b in range(B)]).astype(np.int32))
    a = dict(cand=cand, U=torch.full((B, G, k), 0.25), ea=torch.zeros((V, r), dtype=torch.bfloat16),
             eb=torch.zeros((V, r), dtype=torch.bfloat16),
             gate=torch.ones((B, G, r), dtype=torch.bfloat16), anchor=torch.tensor([3, 4], dtype=torch.int32))
    path = _check_select(a, "ties")
    assert np.array_equal(path, to64(cand[:, :, 0]))


def _verify_det(zt, drafts, T, seeds, what):
    print(f"[verify-det] {what} logits{tuple(zt.shape)} T={T}", flush=True)
    dev = cuda()
    B, G, V = zt.shape
    d_full = torch.zeros((B, G), dtype=torch.int32)
    d_full[:, :G - 1] = drafts[:, :G - 1]
    res = dfl.spec_verify(zt.to(dev), None, d_full.to(dev), T, seeds=seeds.to(dev))
    torch.cuda.synchronize()
    ref = oracle.spec_verify(to64(zt), None, to64(drafts[:, :G - 1]), f32(T),
                             seeds=to64(seeds).astype(np.uint64))
    j, out, acc = to64(res["accept_len"]), to64(res["out_tokens"]), to64(res["accepted"])
    sd = to64(seeds).astype(np.uint64)
    z_t = to64(zt)
    checked = 0
    for b in range(B):
        near = False
        for r in range(G - 1):
            if acc[b, r] != ref["accepted"][b, r]:
                u = oracle.uniform(int(sd[b]), 0, b, r, 1)
                assert abs(u - min(1.0, ref["ratio"][b, r])) < U_EXEMPT, (b, r)
                near = True
        if near:
            continue
        assert j[b] == ref["accept_len"][b], b
        jj = int(j[b])
        np.testing.assert_array_equal(out[b, :jj], ref["out_tokens"][b, :jj])
        np.testing.assert_array_equal(out[b, jj + 1:], ref["out_tokens"][b, jj + 1:])
        if jj < G - 1:
            assert out[b, jj] != int(drafts[b, jj])  # the rejected draft is never the correction
        if out[b, jj] != ref["out_tokens"][b, jj]:
            u = oracle.uniform(int(sd[b]), 0, b, jj, 2)
            assert draw_boundary_ok(z_t[b, jj], f32(T), u, int(out[b, jj]), int(ref["out_tokens"][b, jj]),
                                    residual_exclude=int(drafts[b, jj]) if jj < G - 1 else None), b
        checked += 1
    assert checked >= B // 2
    return j


@pytest.mark.gpu
def test_selected_drafts_verified_with_point_mass_q():
    """The DFlash 2 chain at the serving shape: top-16 -> selector walk -> sampled
    verification of the walk's drafts (q = point mass at each draft)."""
    a = _inputs(32, 8, 16, 151936, 64, seed=23)
    path, _ = _select_gpu(a)
    seeds = syn.philox_seeds(32, 0)
    j = _verify_det(a["zt"], torch.from_numpy(path.astype(np.int32)), 0.7, seeds, "serving")
    assert j.min() >= 0 and j.max() <= 7


@pytest.mark.gpu
def test_point_mass_verify_accepts_certain_drafts():
    """A draft that holds (almost) all of the target's mass is always accepted."""
    B, G, V = 4, 6, 4096
    zt = torch.full((B, G, V), -30.0)
    drafts = torch.from_numpy(np.random.default_rng(1).integers(0, V, (B, G)).astype(np.int32))
    for b in range(B):
        for r in range(G):
            zt[b, r, int(drafts[b, r])] = 30.0
    j = _verify_det(zt, drafts, 1.0, syn.philox_seeds(B, 7), "certain drafts")
    assert (j == G - 1).all()
