"""The drafting path captured in a HIP graph, through the C ABI: context fusion
into two layers' K/V rings, block attention of both layers over those rings,
top-k with the draft draws, sampled verification with a workspace and the same
verification through the entry point that allocates nothing.  The calls are
recorded on a side stream with every output and workspace passed in (so nothing
allocates while capturing), then the graph is replayed three times with other
eager work of the program, and a synchronisation, between the replays.  The
kernels are deterministic and the inputs do not change, so every replay must
reproduce the eager run bit for bit."""
import numpy as np
import pytest
import torch

import block_drafting_context_amd as dfl
from block_drafting_context_amd import synthetic as syn

pytestmark = pytest.mark.gpu

B, G, HQ, HKV, D, W = 4, 8, 8, 2, 128, 256
N_TAPS, D_TGT, D_MODEL, NL = 5, 256, 512, 2
V, K, T, STEP = 5000, 4, 0.7, 5


def _setup(dev):
    rows = B * G
    ctx = torch.tensor([300, 1000, 64, 4096], dtype=torch.int64, device=dev)
    fz = syn.fuse_inputs(rows, N_TAPS, D_TGT, D_MODEL, NL, HKV, D, 41, device=dev, gain_random=True)
    ring = syn.normal((NL, 2, B, HKV, W, D), 41, "ring", dtype=torch.bfloat16, device=dev)
    row_seq = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(G)
    # the block's rows go to the positions just before each sequence's block
    row_pos = (ctx.repeat_interleave(G) - G + torch.arange(G, device=dev).repeat(B)).clamp(min=0)
    layers = [syn.attention_inputs(B, G, HQ, HKV, D, W, [300, 1000, 64, 4096], 42 + i, device=dev)
              for i in range(NL)]
    zt, zd = syn.logits_pair(B, G, V, 2.0, 1.0, 43, device=dev)
    seeds = syn.philox_seeds(B, 7, device=dev)

    def u8(n):
        return torch.empty(max(n, 1), dtype=torch.uint8, device=dev)

    st = {
        "ctx": ctx, "fz": fz, "ring": ring, "ring0": ring.clone(), "row_seq": row_seq,
        "row_pos": row_pos, "layers": layers, "zt": zt, "zd": zd, "seeds": seeds,
        "h": torch.empty((rows, D_MODEL), dtype=torch.bfloat16, device=dev),
        "attn_out": [torch.empty((B, G, HQ, D), dtype=torch.bfloat16, device=dev) for _ in range(NL)],
        "lse_out": [torch.empty((B, G, HQ), dtype=torch.float32, device=dev) for _ in range(NL)],
        "tk": {"idx": torch.empty((B, G, K), dtype=torch.int32, device=dev),
               "val": torch.empty((B, G, K), dtype=torch.float32, device=dev),
               "lse": torch.empty((B, G), dtype=torch.float64, device=dev),
               "draft": torch.empty((B, G), dtype=torch.int32, device=dev)},
        "vo": {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, G), dtype=torch.int32, device=dev),
               "accepted": torch.empty((B, G - 1), dtype=torch.uint8, device=dev)},
        "vn": {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, G), dtype=torch.int32, device=dev),
               "accepted": torch.empty((B, G - 1), dtype=torch.uint8, device=dev)},
        "ws_fuse": u8(dfl.dflash_context_fuse_workspace_size(rows, N_TAPS, D_TGT, D_MODEL, NL, HKV, D)),
        "ws_attn": u8(dfl.dflash_block_attn_workspace_size(B, G, HQ, HKV, D, W)),
        "ws_topk": u8(dfl.dflash_topk_workspace_size(B, G, V, K)),
        "ws_verify": u8(dfl.spec_verify_workspace_size(B, G, V)),
    }
    return st


def _path(st, stream):
    fz = st["fz"]
    dfl.dflash_context_fuse(fz["x"], fz["w_c"], fz["gain"], 1e-6, fz["w_kv"], st["row_seq"],
                            st["row_pos"], st["ring"], N_TAPS, h_t_out=st["h"],
                            workspace=st["ws_fuse"], stream=stream)
    for i, L in enumerate(st["layers"]):
        dfl.dflash_block_attn(L["q"], L["k_blk"], L["v_blk"], st["ring"][i, 0], st["ring"][i, 1],
                              st["ctx"], out=st["attn_out"][i], lse=st["lse_out"][i],
                              workspace=st["ws_attn"], stream=stream)
    tk = dfl.dflash_topk(st["zd"], K, T, seeds=st["seeds"], step=STEP, outputs=st["tk"],
                         workspace=st["ws_topk"], stream=stream)
    dfl.spec_verify(st["zt"], st["zd"], tk["draft"], T, seeds=st["seeds"], step=STEP,
                    draft_lse=tk["lse"], outputs=st["vo"], workspace=st["ws_verify"], stream=stream)
    dfl.spec_verify_noalloc(st["zt"], st["zd"], tk["draft"], T, st["vn"], seeds=st["seeds"],
                            step=STEP, draft_lse=tk["lse"], stream=stream)


def _results(st):
    out = {"ring": st["ring"].view(torch.int16), "h": st["h"].view(torch.int16)}
    for i in range(NL):
        out[f"attn{i}"] = st["attn_out"][i].view(torch.int16)
        out[f"lse{i}"] = st["lse_out"][i]
    for k, v in st["tk"].items():
        out[f"tk_{k}"] = v
    for k, v in st["vo"].items():
        out[f"vo_{k}"] = v
    for k, v in st["vn"].items():
        out[f"vn_{k}"] = v
    return {k: v.clone() for k, v in out.items()}


def _scramble(st):
    # overwrite every output, and put the rings back, so that a replay has to redo all of it
    st["ring"].copy_(st["ring0"])
    st["h"].fill_(3.0)
    for t in st["attn_out"]:
        t.fill_(-1.0)
    for t in st["lse_out"]:
        t.fill_(-1.0)
    for d in (st["tk"], st["vo"], st["vn"]):
        for t in d.values():
            t.fill_(7)


def test_graph_replays_match_eager_path():
    print("[graph] fuse + 2 attention layers + top-k + spec_verify (+ noalloc) captured", flush=True)
    dev = torch.device("cuda:0")
    st = _setup(dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        _path(st, side)          # eager run on the stream that will be captured
    torch.cuda.synchronize()
    ref = _results(st)
    # the verification outputs of both entry points agree (same kernels)
    for k in ("accept_len", "out_tokens", "accepted"):
        assert torch.equal(ref[f"vo_{k}"], ref[f"vn_{k}"]), k
    _scramble(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _path(st, side)
    torch.cuda.synchronize()
    other = torch.randn((512, 512), device=dev)
    for rep in range(3):
        _scramble(st)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _results(st)
        for k in ref:
            assert torch.equal(got[k], ref[k]), (rep, k)
        # eager work of the program between replays
        other = torch.tanh(other @ other.T / 512.0)
        torch.cuda.synchronize()
    assert bool(torch.isfinite(other).all())
