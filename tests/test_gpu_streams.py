"""Concurrent calls on two streams, through the C ABI.  The library keeps no
state between calls and takes its scratch space from the caller's workspace,
so two calls whose workspaces and outputs do not overlap may run at the same
time on different streams.  Each pair below (attention, top-k, sampled
verification, context fusion into separate rings) is launched on two
default-priority streams without synchronisation between them, several times
in a row, and every result must equal, bit for bit, the same call run alone."""
import pytest
import torch

import block_drafting_context_amd as dfl
from block_drafting_context_amd import synthetic as syn

pytestmark = pytest.mark.gpu

B, G, HQ, HKV, D, W = 8, 8, 40, 8, 128, 1024
V, K, T = 20000, 8, 0.7


def _ws(n, dev):
    return torch.empty(max(n, 1), dtype=torch.uint8, device=dev)


def _attn_case(seed, dev):
    a = syn.attention_inputs(B, G, HQ, HKV, D, W, [100 + 300 * i for i in range(B)], seed, device=dev)
    a["out"] = torch.empty((B, G, HQ, D), dtype=torch.bfloat16, device=dev)
    a["ws"] = _ws(dfl.dflash_block_attn_workspace_size(B, G, HQ, HKV, D, W), dev)
    return a


def _attn(a, stream):
    dfl.dflash_block_attn(a["q"], a["k_blk"], a["v_blk"], a["k_ring"], a["v_ring"], a["ctx_len"],
                          out=a["out"], workspace=a["ws"], stream=stream)


def _rows_case(seed, dev):
    zt, zd = syn.logits_pair(B, G, V, 2.0, 1.0, seed, device=dev)
    c = {"zt": zt, "zd": zd, "seeds": syn.philox_seeds(B, seed, device=dev),
         "tk": {"idx": torch.empty((B, G, K), dtype=torch.int32, device=dev),
                "val": torch.empty((B, G, K), dtype=torch.float32, device=dev),
                "lse": torch.empty((B, G), dtype=torch.float64, device=dev),
                "draft": torch.empty((B, G), dtype=torch.int32, device=dev)},
         "vo": {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
                "out_tokens": torch.empty((B, G), dtype=torch.int32, device=dev),
                "accepted": torch.empty((B, G - 1), dtype=torch.uint8, device=dev)},
         "ws_t": _ws(dfl.dflash_topk_workspace_size(B, G, V, K), dev),
         "ws_v": _ws(dfl.spec_verify_workspace_size(B, G, V), dev)}
    return c


def _rows(c, stream):
    tk = dfl.dflash_topk(c["zd"], K, T, seeds=c["seeds"], step=2, outputs=c["tk"], workspace=c["ws_t"],
                         stream=stream)
    dfl.spec_verify(c["zt"], c["zd"], tk["draft"], T, seeds=c["seeds"], step=2, draft_lse=tk["lse"],
                    outputs=c["vo"], workspace=c["ws_v"], stream=stream)


def _fuse_case(seed, dev):
    rows, n_taps, d_tgt, d_model, nl, nkv, dh, bs, w = 64, 5, 512, 1024, 2, 2, 128, 8, 256
    f = syn.fuse_inputs(rows, n_taps, d_tgt, d_model, nl, nkv, dh, seed, device=dev, gain_random=True)
    f["ring"] = syn.normal((nl, 2, bs, nkv, w, dh), seed, "ring", dtype=torch.bfloat16, device=dev)
    f["ring0"] = f["ring"].clone()
    f["rs"] = (torch.arange(rows, device=dev) % bs).to(torch.int32)
    f["rp"] = (torch.arange(rows, device=dev) // bs + 40 * seed).to(torch.int64)
    f["h"] = torch.empty((rows, d_model), dtype=torch.bfloat16, device=dev)
    f["n_taps"] = n_taps
    f["ws"] = _ws(dfl.dflash_context_fuse_workspace_size(rows, n_taps, d_tgt, d_model, nl, nkv, dh), dev)
    return f


def _fuse_reset(f, stream):
    f["ring"].copy_(f["ring0"])  # on the current stream, before the pair starts


def _fuse_run(f, stream):
    dfl.dflash_context_fuse(f["x"], f["w_c"], f["gain"], 1e-6, f["w_kv"], f["rs"], f["rp"], f["ring"],
                            f["n_taps"], h_t_out=f["h"], workspace=f["ws"], stream=stream)


def _pair(make, run, outputs, reset=None):
    dev = torch.device("cuda:0")
    cases = [make(s, dev) for s in (1, 2)]
    # each call alone, one after the other
    alone = []
    for c in cases:
        if reset:
            reset(c, None)
        run(c, torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        alone.append([t.clone() for t in outputs(c)])
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    for rep in range(3):
        for c in cases:
            for t in outputs(c):
                if t.dtype.is_floating_point:
                    t.fill_(-3.0)
                else:
                    t.fill_(5)
            if reset:  # after the fill: restores inputs that the call updates in place
                reset(c, None)
        torch.cuda.synchronize()
        for c, s in zip(cases, streams):
            s.wait_stream(torch.cuda.current_stream(dev))
            run(c, s)
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            for j, t in enumerate(outputs(c)):
                a, b = t, alone[i][j]
                if a.dtype == torch.bfloat16:
                    a, b = a.view(torch.int16), b.view(torch.int16)
                assert torch.equal(a, b), (rep, i, j)


def test_two_attention_calls_on_two_streams():
    print("[streams] block attention x 2", flush=True)
    _pair(_attn_case, _attn, lambda a: [a["out"]])


def test_two_topk_and_verify_sequences_on_two_streams():
    print("[streams] top-k + sampled verify x 2", flush=True)
    _pair(_rows_case, _rows, lambda c: list(c["tk"].values()) + list(c["vo"].values()))


def test_two_fusion_calls_on_two_streams():
    print("[streams] context fusion x 2 (separate rings)", flush=True)
    _pair(_fuse_case, _fuse_run, lambda f: [f["h"], f["ring"]], reset=_fuse_reset)
