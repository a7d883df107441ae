"""Plain fp64 CPU oracle for the DFlash2 block-drafting hot path.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``block_drafting_context_amd``) never imports it, and the two share no code;
the only thing both sides consume is the seeded input generator module
``block_drafting_context_amd.synthetic``, which holds none of the method's
arithmetic.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over independent
rows); this module compiles it with gcc and marshals numpy arrays.  Every
floating input is converted to float64 first (exact for bf16 and fp32).

What each function follows (pages cited by title and section):

* ``block_attn``   -- "DFlash vs DFlash 2": "DFlash: generate the block all at
  once" and "Conditioning on the target model" (Q_i, K_i, V_i equation);
  window and head layout from the "Beam 1.0 DFlash2" model card, "Model".
* ``topk`` / ``draft_rows`` -- "DFlash vs DFlash 2", "The candidate selector"
  (top-k per position) and "The problem: one expensive token at a time"
  (the drafter proposes y from q).
* ``spec_verify`` / ``sampled_verify_seq_u`` -- "DFlash vs DFlash 2", "The
  problem: one expensive token at a time" (greedy prefix match; accept with
  min(1, p/q); residual [p-q]_+; bonus token).
* ``context_fuse`` -- "DFlash vs DFlash 2", "Conditioning on the target
  model" (H_t equation and the context half of K_i, V_i).
* ``position_weights`` -- "DFlash vs DFlash 2", "Training with anchors"
  (w_k equation).
* ``top_p_mask`` -- "Beam 1.0 DFlash2" model card, "Evaluation" (sampled
  runs use temperature 0.7 and top-p 0.99): the nucleus of softmax(z/T)
  kept, everything else masked to -inf.
* ``lm_head_topk`` -- "Beam 1.0 DFlash2" model card, "Model" (the drafter
  reuses the target's LM head) and "DFlash vs DFlash 2", "The candidate
  selector" (top-k per position); top-k, log-normaliser and draft are
  ``draft_rows``' definitions applied to the LM head's logits (one inverse-CDF
  draw over the whole row).
* ``philox4x64_10`` / ``uniform`` -- Salmon et al., SC'11.

Pins: every function is checked by ``tests/test_oracle_*.py`` against values
fixed by the pages or by mathematics (closed forms, invariants, library
routines, exhaustive enumeration); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A different build of oracle.c (the sanitizer test loads one compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer); used as given, never rebuilt.
_LIB_OVERRIDE = os.environ.get("DFLASH_ORACLE_LIB")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)
_I32 = ctypes.POINTER(ctypes.c_int32)
_U64 = ctypes.POINTER(ctypes.c_uint64)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_U16 = ctypes.POINTER(ctypes.c_uint16)


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11",
           "-Wall", "-Wextra", "-o", _LIB_PATH, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if (not os.path.exists(_LIB_PATH)
                or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    c_int, c_i64, c_dbl, c_u64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_uint64
    sigs = {
        "orc_philox4x64_10": (None, [_U64, _U64, _U64]),
        "orc_uniform": (c_dbl, [c_u64] * 5),
        "orc_block_attn": (c_int, [_D, _D, _D, _D, _D, _I64, c_dbl] + [c_int] * 6 + [_D, _D]),
        "orc_topk": (c_int, [_D, c_i64, c_i64, c_int, _I64, _D]),
        "orc_argmax": (c_i64, [_D, c_i64]),
        "orc_logsumexp": (c_dbl, [_D, c_i64, c_dbl]),
        "orc_categorical": (c_i64, [_D, c_i64, c_dbl]),
        "orc_draft_rows": (c_int, [_D, c_int, c_int, c_i64, c_int, c_dbl, _U64, c_u64,
                                   _I64, _D, _D, _I64]),
        "orc_greedy_verify_seq": (c_int, [_D, _I64, c_int, c_i64, _I32, _I64, _U8]),
        "orc_sampled_verify_seq_u": (c_int, [_D, _D, _I64, c_int, c_i64, c_dbl, _D, _D,
                                             _I32, _I64, _U8, _D]),
        "orc_spec_verify": (c_int, [_D, _D, _I64, c_int, c_int, c_i64, c_dbl, _U64, c_u64,
                                    _I32, _I64, _U8, _D]),
        "orc_context_fuse": (c_int, [_D, _D, _D, c_dbl, _D, _I32, _I64] + [c_int] * 8 + [_D, _D]),
        "orc_position_weights": (c_int, [c_int, _D]),
        "orc_select_path": (c_int, [_I64, _D, _D, _D, _D, _I64, c_int, c_int, c_int, c_i64, c_int,
                                    _I64, _D]),
        "orc_two_tap_conv": (c_int, [_D, _D, c_int, c_int, c_int, c_int, _D]),
        "orc_lm_head_topk": (c_int, [_U16, _U16, _I64, c_int, c_int, c_i64, c_int, c_int, c_dbl,
                                     _U64, c_u64, _I64, _D, _D, _I64, _D]),
        "orc_top_p_mask": (c_int, [_D, c_i64, c_i64, c_dbl, c_dbl, _D, _I64]),
        "orc_num_threads": (c_int, []),
        "orc_set_num_threads": (None, [c_int]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (status {rc})")


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    _load().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------- RNG
def philox4x64_10(counter, key) -> np.ndarray:
    lib = _load()
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint64).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64).reshape(2))
    out = np.zeros(4, dtype=np.uint64)
    lib.orc_philox4x64_10(_ptr(c, _U64), _ptr(k, _U64), _ptr(out, _U64))
    return out


def uniform(seed: int, step: int, b: int, row: int, purpose: int) -> float:
    return float(_load().orc_uniform(seed, step, b, row, purpose))


# --------------------------------------------------------------------- attention
def block_attn(q, k_blk, v_blk, k_ring, v_ring, ctx_len, scale, want_lse=False):
    """q [B,G,HQ,D], k_blk/v_blk [B,G,HKV,D], k_ring/v_ring [B,HKV,W,D], ctx_len [B].

    Returns out [B,G,HQ,D] (float64) and, if asked, lse [B,G,HQ]."""
    lib = _load()
    q, kb, vb, kr, vr = (_f64(a) for a in (q, k_blk, v_blk, k_ring, v_ring))
    cl = _i64(ctx_len)
    B, G, HQ, D = q.shape
    HKV = kb.shape[2]
    W = kr.shape[2]
    assert kb.shape == (B, G, HKV, D) and vb.shape == kb.shape
    assert kr.shape == (B, HKV, W, D) and vr.shape == kr.shape and cl.shape == (B,)
    out = np.zeros((B, G, HQ, D), dtype=np.float64)
    lse = np.zeros((B, G, HQ), dtype=np.float64) if want_lse else None
    rc = lib.orc_block_attn(_ptr(q, _D), _ptr(kb, _D), _ptr(vb, _D), _ptr(kr, _D), _ptr(vr, _D),
                            _ptr(cl, _I64), float(scale), B, G, HQ, HKV, D, W,
                            _ptr(out, _D), _ptr(lse, _D))
    _check(rc, "block_attn")
    return (out, lse) if want_lse else out


# ---------------------------------------------------------------- top-k / draws
def topk(z, k):
    """z [..., V] -> (idx int64 [..., k], val float64 [..., k])."""
    lib = _load()
    z = _f64(z)
    V = z.shape[-1]
    rows = int(np.prod(z.shape[:-1])) if z.ndim > 1 else 1
    idx = np.zeros(z.shape[:-1] + (k,), dtype=np.int64)
    val = np.zeros(z.shape[:-1] + (k,), dtype=np.float64)
    _check(lib.orc_topk(_ptr(z, _D), rows, V, int(k), _ptr(idx, _I64), _ptr(val, _D)), "topk")
    return idx, val


def argmax(z) -> int:
    z = _f64(z).reshape(-1)
    return int(_load().orc_argmax(_ptr(z, _D), z.size))


def logsumexp(z, T: float) -> float:
    z = _f64(z).reshape(-1)
    return float(_load().orc_logsumexp(_ptr(z, _D), z.size, float(T)))


def categorical(w, u: float) -> int:
    w = _f64(w).reshape(-1)
    return int(_load().orc_categorical(_ptr(w, _D), w.size, float(u)))


def draft_rows(z, k, temperature, seeds=None, step=0):
    """z [B,G,V] drafter logits -> dict(idx, val, lse, draft)."""
    lib = _load()
    z = _f64(z)
    B, G, V = z.shape
    idx = np.zeros((B, G, k), dtype=np.int64)
    val = np.zeros((B, G, k), dtype=np.float64)
    lse = np.zeros((B, G), dtype=np.float64)
    draft = np.zeros((B, G), dtype=np.int64)
    sd = None if seeds is None else np.ascontiguousarray(np.asarray(seeds, dtype=np.uint64))
    rc = lib.orc_draft_rows(_ptr(z, _D), B, G, V, int(k), float(temperature), _ptr(sd, _U64),
                            int(step), _ptr(idx, _I64), _ptr(val, _D), _ptr(lse, _D),
                            _ptr(draft, _I64))
    _check(rc, "draft_rows")
    return {"idx": idx, "val": val, "lse": lse, "draft": draft}


def lm_head_topk(h_bits, w_bits, gamma, k, temperature, seeds=None, step=0, row_id=None,
                 want_draft=True, want_z=False):
    """Drafter LM head.  h_bits [n, d] and w_bits [V, d] are bf16 bit patterns
    (uint16); row_id [n] global row indices (default 0..n-1), row r belongs to
    sequence r // gamma, block row r % gamma.  Returns dict(idx [n,k], val [n,k],
    lse [n], draft [n] or None, z [n,V] or None)."""
    lib = _load()
    h = np.ascontiguousarray(np.asarray(h_bits, dtype=np.uint16))
    w = np.ascontiguousarray(np.asarray(w_bits, dtype=np.uint16))
    n, d = h.shape
    V = w.shape[0]
    assert w.shape == (V, d)
    rid = None if row_id is None else _i64(row_id).reshape(n)
    sd = None if seeds is None else np.ascontiguousarray(np.asarray(seeds, dtype=np.uint64))
    idx = np.zeros((n, k), dtype=np.int64)
    val = np.zeros((n, k), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    draft = np.zeros(n, dtype=np.int64) if want_draft else None
    z = np.zeros((n, V), dtype=np.float64) if want_z else None
    rc = lib.orc_lm_head_topk(_ptr(h, _U16), _ptr(w, _U16), _ptr(rid, _I64), n, int(gamma), V, d,
                              int(k), float(temperature), _ptr(sd, _U64), int(step),
                              _ptr(idx, _I64), _ptr(val, _D), _ptr(lse, _D), _ptr(draft, _I64),
                              _ptr(z, _D))
    _check(rc, "lm_head_topk")
    return {"idx": idx, "val": val, "lse": lse, "draft": draft, "z": z}


def top_p_mask(z, temperature, top_p):
    """z [..., V] -> (z with the entries outside each row's top-p nucleus set to -inf,
    nucleus sizes [...])."""
    lib = _load()
    z = _f64(z)
    V = z.shape[-1]
    rows = int(np.prod(z.shape[:-1])) if z.ndim > 1 else 1
    out = np.empty_like(z)
    kept = np.zeros(z.shape[:-1] if z.ndim > 1 else (1,), dtype=np.int64)
    _check(lib.orc_top_p_mask(_ptr(z, _D), rows, V, float(temperature), float(top_p),
                              _ptr(out, _D), _ptr(kept, _I64)), "top_p_mask")
    return out, kept


def top_p_cut(z, temperature, top_p):
    """z [..., V] -> (cut_logit [...], cut_index [...], kept [...]): each row's
    top-p nucleus (the one top_p_mask keeps) named by its last entry in the rank
    order (logit descending, index ascending).  Entry v of the row is in the
    nucleus iff z_v > cut_logit, or z_v == cut_logit and v <= cut_index."""
    z = _f64(z)
    V = z.shape[-1]
    rows = z.reshape(-1, V)
    _, kept = top_p_mask(rows, temperature, top_p)
    logit = np.empty(rows.shape[0])
    index = np.empty(rows.shape[0], dtype=np.int64)
    for r in range(rows.shape[0]):
        order = np.lexsort((np.arange(V), -rows[r]))
        last = order[kept[r] - 1]
        logit[r], index[r] = rows[r, last], last
    shape = z.shape[:-1] if z.ndim > 1 else (1,)
    return logit.reshape(shape), index.reshape(shape), kept.reshape(shape)


# ------------------------------------------------------------------------ verify
def sampled_verify_seq_u(zp, zq, drafts, T, u_acc, u_draw):
    """One sequence with explicit uniforms. zp, zq [G,V] (zq None: deterministic
    drafts, q = point mass); drafts [G-1]; u_acc [G-1]; u_draw [G] (u_draw[r] is
    used when the draw is from row r)."""
    lib = _load()
    zp = _f64(zp)
    zq = None if zq is None else _f64(zq)
    G, V = zp.shape
    d = _i64(drafts)
    ua = _f64(u_acc).reshape(-1)
    ud = _f64(u_draw).reshape(-1)
    assert d.shape == (G - 1,) and ua.shape == (G - 1,) and ud.shape == (G,)
    j = np.zeros(1, dtype=np.int32)
    out = np.zeros(G, dtype=np.int64)
    acc = np.zeros(max(G - 1, 1), dtype=np.uint8)
    ratio = np.zeros(max(G - 1, 1), dtype=np.float64)
    rc = lib.orc_sampled_verify_seq_u(_ptr(zp, _D), _ptr(zq, _D), _ptr(d, _I64), G, V, float(T),
                                      _ptr(ua, _D), _ptr(ud, _D), _ptr(j, _I32), _ptr(out, _I64),
                                      _ptr(acc, _U8), _ptr(ratio, _D))
    _check(rc, "sampled_verify_seq_u")
    return {"accept_len": int(j[0]), "out_tokens": out, "accepted": acc[:G - 1],
            "ratio": ratio[:G - 1]}


def spec_verify(zp, zq, drafts, temperature, seeds=None, step=0):
    """zp, zq [B,G,V]; drafts [B,G-1] -> dict(accept_len, out_tokens, accepted, ratio)."""
    lib = _load()
    zp = _f64(zp)
    B, G, V = zp.shape
    zq = None if zq is None else _f64(zq)
    d = _i64(drafts).reshape(B, G - 1)
    sd = None if seeds is None else np.ascontiguousarray(np.asarray(seeds, dtype=np.uint64))
    j = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, G), dtype=np.int64)
    acc = np.zeros((B, max(G - 1, 1)), dtype=np.uint8)
    ratio = np.zeros((B, max(G - 1, 1)), dtype=np.float64)
    rc = lib.orc_spec_verify(_ptr(zp, _D), _ptr(zq, _D), _ptr(d, _I64), B, G, V,
                             float(temperature), _ptr(sd, _U64), int(step), _ptr(j, _I32),
                             _ptr(out, _I64), _ptr(acc, _U8),
                             _ptr(ratio, _D) if temperature > 0 else None)
    _check(rc, "spec_verify")
    return {"accept_len": j, "out_tokens": out, "accepted": acc[:, :G - 1],
            "ratio": ratio[:, :G - 1]}


# -------------------------------------------------------------------- selector
def select_path(cand, score, emb_a, emb_b, gate, anchor):
    """Greedy walk of the candidate selector.  cand [B,G,k] ids; score [B,G,k] = U;
    emb_a, emb_b [V,r]; gate [B,G,r]; anchor [B] -> dict(path [B,G], score [B,G])."""
    lib = _load()
    cand = _i64(cand)
    B, G, k = cand.shape
    score, emb_a, emb_b, gate = _f64(score), _f64(emb_a), _f64(emb_b), _f64(gate)
    V, r = emb_a.shape
    assert score.shape == (B, G, k) and emb_b.shape == (V, r) and gate.shape == (B, G, r)
    anc = _i64(anchor).reshape(B)
    path = np.zeros((B, G), dtype=np.int64)
    ps = np.zeros((B, G), dtype=np.float64)
    rc = lib.orc_select_path(_ptr(cand, _I64), _ptr(score, _D), _ptr(emb_a, _D), _ptr(emb_b, _D),
                             _ptr(gate, _D), _ptr(anc, _I64), B, G, k, V, r, _ptr(path, _I64),
                             _ptr(ps, _D))
    _check(rc, "select_path")
    return {"path": path, "score": ps}


# ------------------------------------------------------------- two-tap conv
def two_tap_conv(x, kern):
    """x [B,G,D]; kern [B,G,2,n_groups] -> y [B,G,D]."""
    lib = _load()
    x, kern = _f64(x), _f64(kern)
    B, G, D = x.shape
    n_groups = kern.shape[3]
    assert kern.shape == (B, G, 2, n_groups)
    y = np.zeros_like(x)
    rc = lib.orc_two_tap_conv(_ptr(x, _D), _ptr(kern, _D), B, G, D, n_groups, _ptr(y, _D))
    _check(rc, "two_tap_conv")
    return y


# ---------------------------------------------------------------------- fusion
def context_fuse(x, wc, g, eps, wkv, row_seq, row_pos, ring, n_layers, n_kv, d_head):
    """x [rows,KX]; wc [DM,KX]; g [DM]; wkv [NL*2*NKV*DH, DM]; ring [NL,2,B,NKV,W,DH]
    (copied, updated and returned).  Returns (h [rows,DM], ring)."""
    lib = _load()
    x, wc, g, wkv = _f64(x), _f64(wc), _f64(g), _f64(wkv)
    ring = _f64(ring).copy()
    rows, KX = x.shape
    DM = wc.shape[0]
    NL, two, B, NKV, W, DH = ring.shape
    assert two == 2 and NL == n_layers and NKV == n_kv and DH == d_head
    assert wc.shape == (DM, KX) and g.shape == (DM,) and wkv.shape == (NL * 2 * NKV * DH, DM)
    rs = np.ascontiguousarray(np.asarray(row_seq, dtype=np.int32))
    rp = _i64(row_pos)
    h = np.zeros((rows, DM), dtype=np.float64)
    rc = lib.orc_context_fuse(_ptr(x, _D), _ptr(wc, _D), _ptr(g, _D), float(eps), _ptr(wkv, _D),
                              _ptr(rs, _I32), _ptr(rp, _I64), rows, KX, DM, NL, NKV, DH, W, B,
                              _ptr(h, _D), _ptr(ring, _D))
    _check(rc, "context_fuse")
    return h, ring


def position_weights(gamma: int) -> np.ndarray:
    w = np.zeros(gamma, dtype=np.float64)
    _check(_load().orc_position_weights(int(gamma), _ptr(w, _D)), "position_weights")
    return w
