"""MI355X (gfx950) DFlash2 block-drafting hot path: Python binding of libdflash.so.

Each function below has the name of the C entry point it wraps (declared in
include/dflash.h) and does argument marshalling only: shape/dtype checks,
output and workspace allocation through torch, and the call on torch's current
HIP stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback.  If the library has not been built (``python -m
block_drafting_context_amd.build``), importing the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "DFlashError", "lib_path", "load", "dflash_status_string", "dflash_version",
    "dflash_block_attn", "dflash_block_attn_workspace_size",
    "dflash_topk", "dflash_topk_workspace_size",
    "spec_verify", "spec_verify_workspace_size",
    "dflash_context_fuse", "dflash_context_fuse_workspace_size",
    "dflash_select_path", "dflash_two_tap_conv",
    "dflash_lm_head_topk", "dflash_lm_head_topk_workspace_size",
    "dflash_top_p_mask", "dflash_top_p_cut", "nucleus_cut_values",
    "spec_verify_noalloc", "spec_verify_noalloc_max_scratch",
    "dflash_device_checks", "dflash_violations",
    "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIB names another build of the same sources (the sanitizer test loads a
# host-only build with AddressSanitizer and UndefinedBehaviorSanitizer).
lib_path = os.environ.get("DFLASH_LIB") or os.path.join(_HERE, "libdflash.so")
_lib = None

EXPORTED_SYMBOLS = (
    "dflash_status_string", "dflash_version",
    "dflash_block_attn_workspace_size", "dflash_block_attn",
    "dflash_topk_workspace_size", "dflash_topk",
    "spec_verify_workspace_size", "spec_verify",
    "dflash_context_fuse_workspace_size", "dflash_context_fuse",
    "dflash_select_path", "dflash_two_tap_conv",
    "dflash_lm_head_topk_workspace_size", "dflash_lm_head_topk",
    "dflash_top_p_mask", "dflash_top_p_cut",
    "spec_verify_noalloc_max_scratch", "spec_verify_noalloc",
    "dflash_device_checks", "dflash_violations",
)
# the same library built with device-data precondition checks
checked_lib_path = os.path.join(_HERE, "libdflash_checked.so")

DTYPE_BF16, DTYPE_FP32 = 0, 1

_vp, _i, _sz, _f, _u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_uint64


class DFlashError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = dflash_status_string(status) if _lib is not None else str(status)
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load():
    """Load libdflash.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"libdflash.so not found at {lib_path}; build it with "
                           "`python -m block_drafting_context_amd.build`")
    lib = ctypes.CDLL(lib_path)
    sig = {
        "dflash_status_string": (ctypes.c_char_p, [_i]),
        "dflash_version": (_i, []),
        "dflash_block_attn_workspace_size": (_sz, [_i] * 7),
        "dflash_block_attn": (_i, [_vp] * 6 + [_f, _vp, _vp, _i] + [_i] * 6 + [_vp, _sz, _vp]),
        "dflash_topk_workspace_size": (_sz, [_i] * 4),
        "dflash_topk": (_i, [_vp, _vp, _i, _i, _i, _i, _f, _vp, _u64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "spec_verify_workspace_size": (_sz, [_i] * 3),
        "spec_verify": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _u64, _vp, _vp, _vp, _i, _i, _i,
                             _vp, _sz, _vp]),
        "dflash_context_fuse_workspace_size": (_sz, [_i] * 7),
        "dflash_context_fuse": (_i, [_vp, _vp, _vp, _f, _vp, _vp, _vp, _vp, _vp] + [_i] * 9 +
                                [_vp, _sz, _vp]),
        "dflash_select_path": (_i, [_vp] * 8 + [_i] * 5 + [_vp]),
        "dflash_two_tap_conv": (_i, [_vp] * 3 + [_i] * 4 + [_vp]),
        "dflash_lm_head_topk_workspace_size": (_sz, [_i] * 4),
        "dflash_top_p_mask": (_i, [_vp, _vp, _vp, _i, _i, _f, _f, _vp]),
        "dflash_top_p_cut": (_i, [_vp, _vp, _vp, _i, _i, _f, _f, _vp]),
        "dflash_device_checks": (_i, []),
        "dflash_violations": (_i, [_vp, _i, _vp]),
        "dflash_lm_head_topk": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _u64, _vp, _vp, _vp,
                                     _vp, _vp, _sz, _vp]),
        "spec_verify_noalloc_max_scratch": (_sz, []),
        "spec_verify_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _u64, _vp, _vp, _vp, _i, _i, _i,
                                     _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def dflash_status_string(status: int) -> str:
    return load().dflash_status_string(int(status)).decode()


def dflash_version() -> int:
    return int(load().dflash_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, None, device)
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace too small: {workspace.numel()} < {nbytes}")
    return workspace, workspace.numel()


def _call(fn_name, *args):
    rc = getattr(load(), fn_name)(*args)
    if rc != 0:
        raise DFlashError(fn_name, rc)


# ------------------------------------------------------------------ attention
def dflash_block_attn_workspace_size(batch, gamma, n_q, n_kv, d_head, window, dtype=DTYPE_BF16):
    return int(load().dflash_block_attn_workspace_size(batch, gamma, n_q, n_kv, d_head, window,
                                                       dtype))


def dflash_block_attn(q, k_blk, v_blk, k_ring, v_ring, ctx_len, scale=None, out=None,
                      want_lse=False, lse=None, workspace=None, stream=None):
    """Block-draft attention of one draft layer.

    q [B,G,HQ,D]; k_blk, v_blk [B,G,HKV,D]; k_ring, v_ring [B,HKV,W,D] (bf16 or
    fp32, all the same); ctx_len [B] int64.  Returns out [B,G,HQ,D] (and lse
    [B,G,HQ] fp32 if asked)."""
    B, G, HQ, D = q.shape
    HKV = k_blk.shape[2]
    W = k_ring.shape[2]
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    dev = q.device
    for t, n, s in ((q, "q", (B, G, HQ, D)), (k_blk, "k_blk", (B, G, HKV, D)),
                    (v_blk, "v_blk", (B, G, HKV, D)), (k_ring, "k_ring", (B, HKV, W, D)),
                    (v_ring, "v_ring", (B, HKV, W, D))):
        _need(t, n, dt, s, dev)
    _need(ctx_len, "ctx_len", torch.int64, (B,), dev)
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    dtype_code = DTYPE_BF16 if dt == torch.bfloat16 else DTYPE_FP32
    if out is None:
        out = torch.empty((B, G, HQ, D), dtype=dt, device=dev)
    _need(out, "out", dt, (B, G, HQ, D), dev)
    if want_lse and lse is None:
        lse = torch.empty((B, G, HQ), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, G, HQ), dev)
    ws, wsb = _workspace(dflash_block_attn_workspace_size(B, G, HQ, HKV, D, W, dtype_code), dev,
                         workspace)
    _call("dflash_block_attn", _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_ring), _ptr(v_ring),
          _ptr(ctx_len), float(scale), _ptr(out), _ptr(lse), dtype_code, B, G, HQ, HKV, D, W,
          _ptr(ws), wsb, _stream(stream))
    return (out, lse) if lse is not None else out


# ---------------------------------------------------------------------- top-k
def dflash_topk_workspace_size(batch, gamma, vocab, k):
    return int(load().dflash_topk_workspace_size(batch, gamma, vocab, k))


def dflash_topk(logits, k, temperature, seeds=None, step=0, outputs=None, workspace=None,
                stream=None, cut=None):
    """Drafter rows: logits [B,G,V] fp32 -> dict(idx [B,G,k] int32, val [B,G,k] fp32,
    lse [B,G] fp64, draft [B,G] int32).  seeds: [B] int64 (bits read as uint64).
    cut: [B,G,2] int32 nucleus cuts from dflash_top_p_cut (top-p), or None."""
    B, G, V = logits.shape
    dev = logits.device
    _need(logits, "logits", torch.float32, (B, G, V), dev)
    if cut is not None:
        _need(cut, "cut", torch.int32, (B, G, 2), dev)
    if seeds is not None:
        _need(seeds, "seeds", torch.int64, (B,), dev)
    o = outputs or {}
    idx = o.get("idx") if o.get("idx") is not None else torch.empty((B, G, k), dtype=torch.int32, device=dev)
    val = o.get("val") if o.get("val") is not None else torch.empty((B, G, k), dtype=torch.float32, device=dev)
    lse = o.get("lse") if o.get("lse") is not None else torch.empty((B, G), dtype=torch.float64, device=dev)
    draft = o.get("draft") if o.get("draft") is not None else torch.empty((B, G), dtype=torch.int32, device=dev)
    _need(idx, "idx", torch.int32, (B, G, k), dev)
    _need(val, "val", torch.float32, (B, G, k), dev)
    _need(lse, "lse", torch.float64, (B, G), dev)
    _need(draft, "draft", torch.int32, (B, G), dev)
    ws, wsb = _workspace(dflash_topk_workspace_size(B, G, V, k), dev, workspace)
    _call("dflash_topk", _ptr(logits), _ptr(cut), B, G, V, int(k), float(temperature), _ptr(seeds),
          int(step), _ptr(idx), _ptr(val), _ptr(lse), _ptr(draft), _ptr(ws), wsb, _stream(stream))
    return {"idx": idx, "val": val, "lse": lse, "draft": draft}


# --------------------------------------------------------------------- verify
def spec_verify_workspace_size(batch, gamma, vocab):
    return int(load().spec_verify_workspace_size(batch, gamma, vocab))


def spec_verify(target_logits, draft_logits, draft_tokens, temperature, seeds=None, step=0,
                draft_lse=None, outputs=None, workspace=None, stream=None, target_cut=None,
                draft_cut=None):
    """target_logits, draft_logits [B,G,V] fp32 (draft_logits None with temperature > 0:
    deterministic drafts, e.g. from dflash_select_path); draft_tokens [B,G] int32 (first G-1
    used); draft_lse [B,G] fp64 or None; target_cut, draft_cut [B,G,2] int32 nucleus cuts
    (top-p) or None.  Returns dict(accept_len [B] int32, out_tokens [B,G] int32, accepted
    [B,G-1] uint8)."""
    B, G, V = target_logits.shape
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, (B, G, V), dev)
    _check_cuts(target_cut, draft_cut, B, G, dev)
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, (B, G, V), dev)
    _need(draft_tokens, "draft_tokens", torch.int32, (B, G), dev)
    if draft_lse is not None:
        _need(draft_lse, "draft_lse", torch.float64, (B, G), dev)
    if seeds is not None:
        _need(seeds, "seeds", torch.int64, (B,), dev)
    o = outputs or {}
    acc_len = o.get("accept_len") if o.get("accept_len") is not None else torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = o.get("out_tokens") if o.get("out_tokens") is not None else torch.empty((B, G), dtype=torch.int32, device=dev)
    accepted = o.get("accepted") if o.get("accepted") is not None else torch.empty((B, max(G - 1, 1)), dtype=torch.uint8, device=dev)
    _need(acc_len, "accept_len", torch.int32, (B,), dev)
    _need(out_tok, "out_tokens", torch.int32, (B, G), dev)
    _need(accepted, "accepted", torch.uint8, (B, max(G - 1, 1)), dev)
    ws, wsb = _workspace(spec_verify_workspace_size(B, G, V), dev, workspace)
    _call("spec_verify", _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens),
          _ptr(draft_lse), _ptr(target_cut), _ptr(draft_cut), float(temperature), _ptr(seeds), int(step), _ptr(acc_len),
          _ptr(out_tok), _ptr(accepted), B, G, V, _ptr(ws), wsb, _stream(stream))
    return {"accept_len": acc_len, "out_tokens": out_tok, "accepted": accepted[:, :G - 1]}


def _check_cuts(target_cut, draft_cut, B, G, dev):
    if target_cut is not None:
        _need(target_cut, "target_cut", torch.int32, (B, G, 2), dev)
    if draft_cut is not None:
        _need(draft_cut, "draft_cut", torch.int32, (B, G, 2), dev)


def spec_verify_noalloc_max_scratch():
    return int(load().spec_verify_noalloc_max_scratch())


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, temperature, outputs,
                        seeds=None, step=0, draft_lse=None, stream=None, target_cut=None,
                        draft_cut=None):
    """spec_verify with the library's static per-GPU scratch instead of a workspace: the
    call allocates nothing, so the caller passes every output (dict accept_len [B] int32,
    out_tokens [B,G] int32, accepted [B,G-1] uint8).  Calls that overlap on one GPU race."""
    B, G, V = target_logits.shape
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, (B, G, V), dev)
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, (B, G, V), dev)
    _need(draft_tokens, "draft_tokens", torch.int32, (B, G), dev)
    if draft_lse is not None:
        _need(draft_lse, "draft_lse", torch.float64, (B, G), dev)
    if seeds is not None:
        _need(seeds, "seeds", torch.int64, (B,), dev)
    _check_cuts(target_cut, draft_cut, B, G, dev)
    acc_len, out_tok, accepted = outputs["accept_len"], outputs["out_tokens"], outputs["accepted"]
    _need(acc_len, "accept_len", torch.int32, (B,), dev)
    _need(out_tok, "out_tokens", torch.int32, (B, G), dev)
    _need(accepted, "accepted", torch.uint8, (B, max(G - 1, 1)), dev)
    _call("spec_verify_noalloc", _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens),
          _ptr(draft_lse), _ptr(target_cut), _ptr(draft_cut), float(temperature), _ptr(seeds), int(step), _ptr(acc_len),
          _ptr(out_tok), _ptr(accepted), B, G, V, _stream(stream))
    return outputs


# ------------------------------------------------------------------- selector
def dflash_select_path(cand_idx, cand_score, emb_a, emb_b, gate, anchor, path=None,
                       path_score=None, stream=None):
    """cand_idx [B,G,k] int32; cand_score [B,G,k] fp32; emb_a, emb_b [V,r] bf16; gate [B,G,r]
    bf16; anchor [B] int32.  Returns dict(path [B,G] int32, score [B,G] fp32)."""
    B, G, k = cand_idx.shape
    V, r = emb_a.shape
    dev = cand_idx.device
    _need(cand_idx, "cand_idx", torch.int32, (B, G, k), dev)
    _need(cand_score, "cand_score", torch.float32, (B, G, k), dev)
    _need(emb_a, "emb_a", torch.bfloat16, (V, r), dev)
    _need(emb_b, "emb_b", torch.bfloat16, (V, r), dev)
    _need(gate, "gate", torch.bfloat16, (B, G, r), dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    path = path if path is not None else torch.empty((B, G), dtype=torch.int32, device=dev)
    score = path_score if path_score is not None else torch.empty((B, G), dtype=torch.float32,
                                                                  device=dev)
    _need(path, "path", torch.int32, (B, G), dev)
    _need(score, "path_score", torch.float32, (B, G), dev)
    _call("dflash_select_path", _ptr(cand_idx), _ptr(cand_score), _ptr(emb_a), _ptr(emb_b),
          _ptr(gate), _ptr(anchor), _ptr(path), _ptr(score), B, G, k, V, r, _stream(stream))
    return {"path": path, "score": score}


# ------------------------------------------------------------- two-tap conv
def dflash_two_tap_conv(x, kern, y=None, stream=None):
    """x [B,G,D] bf16; kern [B,G,2,n_groups] fp32 -> y [B,G,D] bf16 (y must not be x)."""
    B, G, D = x.shape
    n_groups = kern.shape[3]
    dev = x.device
    _need(x, "x", torch.bfloat16, (B, G, D), dev)
    _need(kern, "kern", torch.float32, (B, G, 2, n_groups), dev)
    y = y if y is not None else torch.empty_like(x)
    _need(y, "y", torch.bfloat16, (B, G, D), dev)
    _call("dflash_two_tap_conv", _ptr(x), _ptr(kern), _ptr(y), B, G, D, n_groups, _stream(stream))
    return y


# ---------------------------------------------------------------------- top-p
def dflash_top_p_mask(logits, temperature, top_p, out=None, want_kept=False, stream=None):
    """logits [..., V] fp32 -> (rows with the entries outside each row's top-p nucleus
    set to -inf, nucleus sizes [...] int32 or None).  out=logits masks in place."""
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    dev = logits.device
    _need(logits, "logits", torch.float32, None, dev)
    out = out if out is not None else torch.empty_like(logits)
    _need(out, "out", torch.float32, tuple(logits.shape), dev)
    kept = torch.empty(logits.shape[:-1], dtype=torch.int32, device=dev) if want_kept else None
    _call("dflash_top_p_mask", _ptr(logits), _ptr(out), _ptr(kept), rows, V, float(temperature),
          float(top_p), _stream(stream))
    return out, kept


def dflash_top_p_cut(logits, temperature, top_p, cut=None, want_kept=False, stream=None):
    """logits [..., V] fp32 -> (nucleus cuts [..., 2] int32: the bits of the last nucleus
    entry's logit, then its index; nucleus sizes [...] int32 or None).  The cuts go to
    dflash_topk(cut=...) and spec_verify(target_cut=..., draft_cut=...)."""
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    dev = logits.device
    _need(logits, "logits", torch.float32, None, dev)
    shape = tuple(logits.shape[:-1]) + (2,)
    cut = cut if cut is not None else torch.empty(shape, dtype=torch.int32, device=dev)
    _need(cut, "cut", torch.int32, shape, dev)
    kept = torch.empty(logits.shape[:-1], dtype=torch.int32, device=dev) if want_kept else None
    _call("dflash_top_p_cut", _ptr(logits), _ptr(cut), _ptr(kept), rows, V, float(temperature),
          float(top_p), _stream(stream))
    return cut, kept


def nucleus_cut_values(cut):
    """Cuts [..., 2] int32 -> (logit [...] fp32, index [...] int32): entry v of the row is
    in the nucleus iff z_v > logit, or z_v == logit and v <= index."""
    return cut[..., 0].view(torch.float32), cut[..., 1]


# ------------------------------------------------------------ device checks
def dflash_device_checks():
    """1 when the loaded library records violated device-data preconditions."""
    return int(load().dflash_device_checks())


def dflash_violations(clear=True, stream=None):
    """The DFLASH_VIOLATION_* bits recorded on the current GPU (after `stream`);
    raises DFlashError(-3) in a release build."""
    word = ctypes.c_uint32(0)
    st = _stream(stream) if dflash_device_checks() else None  # a release build makes no HIP call
    _call("dflash_violations", ctypes.byref(word), int(bool(clear)), st)
    return int(word.value)


# -------------------------------------------------------------------- LM head
def dflash_lm_head_topk_workspace_size(rows, d_model, vocab, k):
    return int(load().dflash_lm_head_topk_workspace_size(rows, d_model, vocab, k))


def dflash_lm_head_topk(hidden, w_head, gamma, k, temperature, seeds=None, step=0,
                        want_lse=True, want_draft=True, outputs=None, workspace=None,
                        stream=None):
    """Drafter LM head with fused top-k: hidden [rows, d] bf16; w_head [V, d] bf16 ->
    dict(idx [rows,k] int32, val [rows,k] fp32, lse [rows] fp64 or None, draft [rows]
    int32 or None).  Row r belongs to sequence r // gamma; seeds [ceil(rows/gamma)]
    int64 (bits read as uint64)."""
    rows, d = hidden.shape
    V = w_head.shape[0]
    dev = hidden.device
    _need(hidden, "hidden", torch.bfloat16, (rows, d), dev)
    _need(w_head, "w_head", torch.bfloat16, (V, d), dev)
    if seeds is not None:
        _need(seeds, "seeds", torch.int64, ((rows + gamma - 1) // gamma,), dev)
    o = outputs or {}
    idx = o.get("idx") if o.get("idx") is not None else torch.empty((rows, k), dtype=torch.int32, device=dev)
    val = o.get("val") if o.get("val") is not None else torch.empty((rows, k), dtype=torch.float32, device=dev)
    lse = o.get("lse") if o.get("lse") is not None else (
        torch.empty(rows, dtype=torch.float64, device=dev) if want_lse else None)
    draft = o.get("draft") if o.get("draft") is not None else (
        torch.empty(rows, dtype=torch.int32, device=dev) if want_draft else None)
    _need(idx, "idx", torch.int32, (rows, k), dev)
    _need(val, "val", torch.float32, (rows, k), dev)
    if lse is not None:
        _need(lse, "lse", torch.float64, (rows,), dev)
    if draft is not None:
        _need(draft, "draft", torch.int32, (rows,), dev)
    ws, wsb = _workspace(dflash_lm_head_topk_workspace_size(rows, d, V, k), dev, workspace)
    _call("dflash_lm_head_topk", _ptr(hidden), _ptr(w_head), rows, int(gamma), d, V, int(k),
          float(temperature), _ptr(seeds), int(step), _ptr(idx), _ptr(val), _ptr(lse),
          _ptr(draft), _ptr(ws), wsb, _stream(stream))
    return {"idx": idx, "val": val, "lse": lse, "draft": draft}


# --------------------------------------------------------------------- fusion
def dflash_context_fuse_workspace_size(rows, n_taps, d_tgt, d_model, n_layers, n_kv, d_head):
    return int(load().dflash_context_fuse_workspace_size(rows, n_taps, d_tgt, d_model, n_layers,
                                                         n_kv, d_head))


def dflash_context_fuse(taps, w_c, rms_gain, eps, w_kv, row_seq, row_pos, kv_ring, n_taps,
                        h_t_out=None, workspace=None, stream=None):
    """taps [rows, n_taps*d_tgt] bf16; w_c [d_model, n_taps*d_tgt] bf16; rms_gain [d_model]
    fp32; w_kv [n_layers*2*n_kv*d_head, d_model] bf16; row_seq [rows] int32; row_pos [rows]
    int64; kv_ring [n_layers, 2, B, n_kv, W, d_head] bf16 (updated in place)."""
    rows, kx = taps.shape
    d_model = w_c.shape[0]
    NL, two, B, NKV, W, DH = kv_ring.shape
    dev = taps.device
    if two != 2 or kx % n_taps:
        raise ValueError("bad shapes")
    _need(taps, "taps", torch.bfloat16, (rows, kx), dev)
    _need(w_c, "w_c", torch.bfloat16, (d_model, kx), dev)
    _need(rms_gain, "rms_gain", torch.float32, (d_model,), dev)
    _need(w_kv, "w_kv", torch.bfloat16, (NL * 2 * NKV * DH, d_model), dev)
    _need(row_seq, "row_seq", torch.int32, (rows,), dev)
    _need(row_pos, "row_pos", torch.int64, (rows,), dev)
    _need(kv_ring, "kv_ring", torch.bfloat16, None, dev)
    if h_t_out is not None:
        _need(h_t_out, "h_t_out", torch.bfloat16, (rows, d_model), dev)
    ws, wsb = _workspace(dflash_context_fuse_workspace_size(rows, n_taps, kx // n_taps, d_model,
                                                            NL, NKV, DH), dev, workspace)
    _call("dflash_context_fuse", _ptr(taps), _ptr(w_c), _ptr(rms_gain), float(eps), _ptr(w_kv),
          _ptr(row_seq), _ptr(row_pos), _ptr(kv_ring), _ptr(h_t_out), rows, n_taps, kx // n_taps,
          d_model, NL, NKV, DH, W, B, _ptr(ws), wsb, _stream(stream))
    return kv_ring
