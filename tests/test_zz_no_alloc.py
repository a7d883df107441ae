"""spec_verify_noalloc (the verification with the library's static per-GPU
scratch, for callers that cannot allocate) against spec_verify on the same
inputs, through the C ABI: two calls in a row, the second smaller, at the
throughput shape and small shapes, greedy, sampled, sampled with the draft
normaliser given, deterministic drafts, and top-p nucleus cuts on both sides.  Both entry points run the same
kernels, so the outputs must be identical."""
import numpy as np
import pytest
import torch

import block_drafting_context_amd as dfl
from block_drafting_context_amd import synthetic as syn

pytestmark = pytest.mark.gpu


def _outputs(B, G, dev):
    # fill with garbage first: every entry must be overwritten
    return {"accept_len": torch.full((B,), -7, dtype=torch.int32, device=dev),
            "out_tokens": torch.full((B, G), -7, dtype=torch.int32, device=dev),
            "accepted": torch.full((B, max(G - 1, 1)), 7, dtype=torch.uint8, device=dev)}


def _case(B, G, V, T, mode, seed):
    print(f"[noalloc] B={B} G={G} V={V} T={T} mode={mode}", flush=True)
    dev = torch.device("cuda:0")
    zt, zd = syn.logits_pair(B, G, V, 2.0, 1.0, seed=seed)
    zt, zd = zt.to(dev), zd.to(dev)
    seeds = syn.philox_seeds(B, seed).to(dev) if T > 0 else None
    tc = dc = None
    if mode == "top_p":  # nucleus cuts on both sides
        tc, _ = dfl.dflash_top_p_cut(zt, T, 0.95)
        dc, _ = dfl.dflash_top_p_cut(zd, T, 0.95)
    tk = dfl.dflash_topk(zd, 4, T, seeds=seeds, step=3, cut=dc)
    drafts = tk["draft"]
    dl = None if mode == "deterministic" else zd
    lse = tk["lse"] if mode in ("with_lse", "top_p") else None
    ref = dfl.spec_verify(zt, dl, drafts, T, seeds=seeds, step=3, draft_lse=lse, target_cut=tc,
                          draft_cut=dc)
    got = dfl.spec_verify_noalloc(zt, dl, drafts, T, _outputs(B, G, dev), seeds=seeds, step=3,
                                  draft_lse=lse, target_cut=tc, draft_cut=dc)
    torch.cuda.synchronize()
    for key in ("accept_len", "out_tokens"):
        assert torch.equal(got[key].cpu(), ref[key].cpu()), key
    assert torch.equal(got["accepted"][:, :G - 1].cpu(), ref["accepted"].cpu())


@pytest.mark.parametrize("mode", ["sampled", "with_lse", "deterministic", "top_p"])
def test_noalloc_matches_spec_verify_twice_second_smaller(mode):
    _case(32, 8, 151936, 0.7, mode, seed=11)
    _case(3, 5, 5000, 0.9, mode, seed=12)


def test_noalloc_greedy_twice_second_smaller():
    _case(16, 16, 151936, 0.0, "sampled", seed=13)
    _case(2, 4, 1024, 0.0, "sampled", seed=14)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    dev = torch.device("cuda:0")
    cap = dfl.spec_verify_noalloc_max_scratch()
    B, G, V = 1024, 32, 151936
    assert dfl.spec_verify_workspace_size(B, G, V) > cap
    zt = torch.empty((B, G, 4), dtype=torch.float32, device=dev)  # never read: rejected first
    with pytest.raises(dfl.DFlashError) as e:
        dfl._call("spec_verify_noalloc", dfl._ptr(zt), None, dfl._ptr(zt), None, None, None, 0.0, None, 0,
                  dfl._ptr(zt), dfl._ptr(zt), None, B, G, V, None)
    assert e.value.status == -6
