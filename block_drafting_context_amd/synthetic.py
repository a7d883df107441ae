"""Seeded synthetic inputs for the block-drafting hot path.

This module only draws random tensors of the right shapes, dtypes and value
distributions; it holds none of the method's arithmetic.  Both the GPU path
(tests, benchmark) and the CPU oracle consume what it produces: the GPU gets
the tensors, the oracle gets exact float64 copies of the same values.

Every tensor is drawn from its own torch generator, seeded from
(workload seed, tensor name) through numpy's SeedSequence, so any tensor can be
regenerated on its own and on any device.  bf16 tensors are drawn in fp32 and
rounded to nearest-even.
"""
from __future__ import annotations

import zlib

import numpy as np
import torch


def _seed(seed: int, name: str) -> int:
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=(zlib.crc32(name.encode()),))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def generator(seed: int, name: str, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, name))
    return g


def normal(shape, seed: int, name: str, std=1.0, mean=0.0, dtype=torch.float32, device="cpu"):
    """N(mean, std^2) samples drawn in fp32, then cast (bf16: round-to-nearest-even)."""
    g = generator(seed, name, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(dtype)


def uniform_int(shape, lo: int, hi: int, seed: int, name: str, device="cpu"):
    """Integers uniform on [lo, hi] inclusive (int64)."""
    g = generator(seed, name, device)
    return torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device, dtype=torch.int64)


def ctx_lengths(batch: int, lo: int, hi: int, seed: int, device="cpu"):
    """Per-sequence total context length, uniform on [lo, hi]."""
    return uniform_int((batch,), lo, hi, seed, "ctx_len", device)


def attention_inputs(batch, gamma, n_q, n_kv, d_head, window, ctx_len, seed,
                     dtype=torch.bfloat16, device="cpu", q_mult=1.0, k_std=None,
                     v_mean=0.0, poison_invalid=False):
    """Q [B,G,HQ,D], block K/V [B,G,HKV,D], ring K/V [B,HKV,W,D] ~ N(0,1)/sqrt(D).

    q_mult scales Q (score-spread stress case); k_std overrides the K std;
    v_mean shifts V (accumulation-precision stress case); poison_invalid fills
    ring slots at or beyond min(ctx_len, window) with NaN."""
    std = 1.0 / float(np.sqrt(d_head))
    ks = std if k_std is None else k_std
    q = normal((batch, gamma, n_q, d_head), seed, "q", std=std * q_mult, dtype=dtype, device=device)
    kb = normal((batch, gamma, n_kv, d_head), seed, "k_blk", std=ks, dtype=dtype, device=device)
    vb = normal((batch, gamma, n_kv, d_head), seed, "v_blk", std=std, mean=v_mean, dtype=dtype,
                device=device)
    kr = normal((batch, n_kv, window, d_head), seed, "k_ring", std=ks, dtype=dtype, device=device)
    vr = normal((batch, n_kv, window, d_head), seed, "v_ring", std=std, mean=v_mean, dtype=dtype,
                device=device)
    cl = torch.as_tensor(ctx_len, dtype=torch.int64).to(device).reshape(batch)
    if poison_invalid:
        n = torch.clamp(cl, max=window).to(device)
        slot = torch.arange(window, device=device)
        bad = (slot[None, :] >= n[:, None])[:, None, :, None]
        kr = kr.masked_fill(bad, float("nan"))
        vr = vr.masked_fill(bad, float("nan"))
    return {"q": q, "k_blk": kb, "v_blk": vb, "k_ring": kr, "v_ring": vr, "ctx_len": cl}


def logits_pair(batch, gamma, vocab, target_std, noise_std, seed, device="cpu"):
    """Target logits ~ N(0, target_std^2); drafter = target + N(0, s_r^2) where s_r
    is noise_std (a scalar, or one value per block row)."""
    zt = normal((batch, gamma, vocab), seed, "target_logits", std=target_std, device=device)
    noise = normal((batch, gamma, vocab), seed, "draft_noise", device=device)
    s = torch.as_tensor(noise_std, dtype=torch.float32, device=device)
    if s.ndim == 0:
        zd = zt + noise * s
    else:
        zd = zt + noise * s.reshape(1, gamma, 1)
    return zt.contiguous(), zd.contiguous()


def linear_noise_std(gamma, first, last):
    """Per-row noise std growing linearly from `first` at row 1 to `last` at row gamma."""
    if gamma == 1:
        return np.array([first], dtype=np.float32)
    return np.array([first + (last - first) * r / (gamma - 1) for r in range(gamma)],
                    dtype=np.float32)


def fuse_inputs(rows, n_taps, d_tgt, d_model, n_layers, n_kv, d_head, seed, device="cpu",
                dtype=torch.bfloat16, gain_random=False):
    """Tapped target states ~ N(0,1); W_c ~ N(0, 1/(n_taps*d_tgt)); W_kv ~ N(0, 1/d_model);
    RMSNorm gain = 1 (or ~ U-like N(1, 0.25^2) when gain_random)."""
    kx = n_taps * d_tgt
    nkv = n_layers * 2 * n_kv * d_head
    x = normal((rows, kx), seed, "taps", dtype=dtype, device=device)
    wc = normal((d_model, kx), seed, "w_c", std=1.0 / np.sqrt(kx), dtype=dtype, device=device)
    wkv = normal((nkv, d_model), seed, "w_kv", std=1.0 / np.sqrt(d_model), dtype=dtype,
                 device=device)
    if gain_random:
        g = normal((d_model,), seed, "gain", std=0.25, mean=1.0, device=device)
    else:
        g = torch.ones(d_model, dtype=torch.float32, device=device)
    return {"x": x, "w_c": wc, "w_kv": wkv, "gain": g}


def lm_head_inputs(rows, d_model, vocab, seed, logit_std=5 ** 0.5, device="cpu",
                   dtype=torch.bfloat16):
    """Drafter hidden rows h ~ N(0,1) and LM-head weights W ~ N(0, logit_std^2 / d_model)
    (one row per vocabulary entry), so the logits h W^T are ~ N(0, logit_std^2)."""
    h = normal((rows, d_model), seed, "head_hidden", dtype=dtype, device=device)
    w = normal((vocab, d_model), seed, "w_head", std=logit_std / float(np.sqrt(d_model)),
               dtype=dtype, device=device)
    return h, w


def philox_seeds(batch, base=0, device="cpu"):
    """Per-sequence generator seeds base, base+1, ... as int64 (reinterpreted as uint64)."""
    return torch.arange(base, base + batch, dtype=torch.int64, device=device)
