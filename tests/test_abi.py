"""The C ABI without a GPU: the library loads, exports every entry point that
include/dflash.h declares, answers workspace queries, and rejects every
host-checkable bad argument with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

import block_drafting_context_amd as dfl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")
P = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_symbols_are_exported():
    lib = dfl.load()
    names = declared_functions()
    assert set(names) == set(dfl.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert dfl.dflash_status_string(code) != "unknown status"
    assert dfl.dflash_status_string(17) == "unknown status"
    assert dfl.dflash_version() >= 100


def test_workspace_queries():
    assert dfl.dflash_block_attn_workspace_size(1, 8, 40, 8, 128, 4096) > 0   # split keys at B=1
    assert dfl.dflash_block_attn_workspace_size(32, 8, 40, 8, 128, 4096, 1) == 0  # fp32: none
    assert dfl.dflash_block_attn_workspace_size(32, 8, 41, 8, 128, 4096) == 0      # bad GQA
    assert dfl.dflash_topk_workspace_size(32, 8, 151936, 8) == 0   # all in LDS
    assert dfl.spec_verify_workspace_size(32, 8, 151936) > 0
    assert dfl.dflash_context_fuse_workspace_size(512, 5, 5120, 5120, 5, 8, 128) > 0
    assert dfl.dflash_context_fuse_workspace_size(512, 5, 5120, 5100, 5, 8, 128) == 0


def attn(**kw):
    a = dict(q=P, kb=P, vb=P, kr=P, vr=P, cl=P, scale=0.1, out=P, lse=None, dtype=0, B=2, G=8,
             HQ=40, HKV=8, D=128, W=4096, ws=None, wsb=0, st=None)
    a.update(kw)
    return dfl.load().dflash_block_attn(a["q"], a["kb"], a["vb"], a["kr"], a["vr"], a["cl"],
                                        a["scale"], a["out"], a["lse"], a["dtype"], a["B"], a["G"],
                                        a["HQ"], a["HKV"], a["D"], a["W"], a["ws"], a["wsb"],
                                        a["st"])


def test_block_attn_validation():
    assert attn(q=None) == -1
    assert attn(out=None) == -1
    assert attn(HQ=41) == -2
    assert attn(G=0) == -2
    assert attn(scale=0.0) == -2
    assert attn(scale=float("nan")) == -2
    assert attn(dtype=7) == -2
    assert attn(G=33) == -3
    assert attn(D=96) == -3
    assert attn(W=4000) == -3
    assert attn(B=1) == -4         # needs a workspace at this size
    assert attn(ws=ctypes.c_void_p(0x1001), wsb=1 << 30) == -4  # misaligned
    assert attn(B=0) == 0           # nothing to do, nothing launched


def topk(**kw):
    a = dict(z=P, cut=None, B=2, G=8, V=151936, k=8, T=0.7, seeds=P, step=0, idx=P, val=P,
             lse=None, draft=P, ws=None, wsb=0, st=None)
    a.update(kw)
    return dfl.load().dflash_topk(a["z"], a["cut"], a["B"], a["G"], a["V"], a["k"], a["T"], a["seeds"],
                                  a["step"], a["idx"], a["val"], a["lse"], a["draft"], a["ws"],
                                  a["wsb"], a["st"])


def test_topk_validation():
    assert topk(z=None) == -1
    assert topk(seeds=None) == -1          # sampling needs seeds
    assert topk(k=0) == -2
    assert topk(k=151937) == -2
    assert topk(T=-1.0) == -2
    assert topk(T=float("inf")) == -2
    assert topk(k=65) == -3
    assert topk(V=151935) == -3
    assert topk(V=(1 << 29) + 4) == -3     # row bytes past 32-bit buffer offsets
    assert topk(V=(1 << 23) + 4) == -3     # segment statistics past the workgroup's LDS
    assert topk(G=40) == -3
    assert topk(seeds=None, T=0.0, k=65) == -3  # greedy needs no seeds: fails on k only


def verify(**kw):
    a = dict(zp=P, zq=P, d=P, lse=None, tc=None, dc=None, T=0.7, seeds=P, step=0, j=P, out=P,
             acc=None, B=2, G=8, V=151936, ws=None, wsb=0, st=None)
    a.update(kw)
    return dfl.load().spec_verify(a["zp"], a["zq"], a["d"], a["lse"], a["tc"], a["dc"], a["T"], a["seeds"],
                                  a["step"], a["j"], a["out"], a["acc"], a["B"], a["G"], a["V"],
                                  a["ws"], a["wsb"], a["st"])


def test_verify_validation():
    assert verify(zp=None) == -1
    assert verify(zq=None) == -4  # no draft logits at T > 0: deterministic drafts; then workspace
    assert verify(seeds=None) == -1
    assert verify(j=None) == -1
    assert verify(G=0) == -2
    assert verify(T=-0.5) == -2
    assert verify(G=33) == -3
    assert verify(V=1001) == -3
    assert verify(V=(1 << 29) + 4) == -3
    assert verify() == -4
    assert verify(zq=None, seeds=None, T=0.0) == -4


def select(**kw):
    a = dict(c=P, u=P, ea=P, eb=P, g=P, anc=P, path=P, ps=None, B=32, G=8, k=16, V=151936, r=64,
             st=None)
    a.update(kw)
    return dfl.load().dflash_select_path(a["c"], a["u"], a["ea"], a["eb"], a["g"], a["anc"],
                                         a["path"], a["ps"], a["B"], a["G"], a["k"], a["V"], a["r"],
                                         a["st"])


def test_select_path_validation():
    assert select(B=0) == 0
    assert select(c=None) == -1
    assert select(anc=None) == -1
    assert select(path=None) == -1
    assert select(G=0) == -2
    assert select(k=0) == -2
    assert select(r=0) == -2
    assert select(k=65) == -3
    assert select(r=60) == -3
    assert select(ea=ctypes.c_void_p(0x1008)) == -3  # rows must be 16-byte aligned


def conv(**kw):
    a = dict(x=P, k=P, y=ctypes.c_void_p(0x2000), B=32, G=8, d=5120, ng=80, st=None)
    a.update(kw)
    return dfl.load().dflash_two_tap_conv(a["x"], a["k"], a["y"], a["B"], a["G"], a["d"], a["ng"],
                                          a["st"])


def test_two_tap_conv_validation():
    assert conv(B=0) == 0
    assert conv(x=None) == -1
    assert conv(k=None) == -1
    assert conv(G=0) == -2
    assert conv(ng=3) == -2          # groups must divide the width
    assert conv(y=P) == -2           # in place is not allowed
    assert conv(ng=1024) == -3       # groups of 5 channels: not a multiple of 8
    assert conv(x=ctypes.c_void_p(0x1008)) == -3


def fuse(**kw):
    a = dict(x=P, wc=P, g=P, eps=1e-6, wkv=P, rs=P, rp=P, ring=P, h=None, rows=512, taps=5,
             dt=5120, dm=5120, nl=5, nkv=8, dh=128, W=4096, B=64, ws=None, wsb=0, st=None)
    a.update(kw)
    return dfl.load().dflash_context_fuse(a["x"], a["wc"], a["g"], a["eps"], a["wkv"], a["rs"],
                                          a["rp"], a["ring"], a["h"], a["rows"], a["taps"], a["dt"],
                                          a["dm"], a["nl"], a["nkv"], a["dh"], a["W"], a["B"],
                                          a["ws"], a["wsb"], a["st"])


def test_fuse_validation():
    assert fuse(x=None) == -1
    assert fuse(ring=None) == -1
    assert fuse(rows=0) == -2
    assert fuse(eps=-1.0) == -2
    assert fuse(dm=5100) == -3
    assert fuse(dm=16384) == -3
    assert fuse(dh=126) == -3
    assert fuse() == -4


def test_binding_raises_on_bad_status():
    with pytest.raises(dfl.DFlashError) as e:
        dfl._call("dflash_topk", P, None, 1, 1, 1024, 0, 0.0, None, 0, P, P, None, None, None, 0, None)
    assert e.value.status == -2


def head(**kw):
    a = dict(h=P, w=P, rows=256, G=8, d=5120, V=151936, k=8, T=0.7, seeds=P, step=0, idx=P,
             val=P, lse=None, draft=P, ws=None, wsb=0, st=None)
    a.update(kw)
    return dfl.load().dflash_lm_head_topk(a["h"], a["w"], a["rows"], a["G"], a["d"], a["V"], a["k"],
                                          a["T"], a["seeds"], a["step"], a["idx"], a["val"],
                                          a["lse"], a["draft"], a["ws"], a["wsb"], a["st"])


def test_lm_head_validation():
    assert head(rows=0) == 0                 # nothing to do, nothing launched
    assert head(rows=-1) == -2
    assert head(G=0) == -2
    assert head(k=0) == -2
    assert head(V=4, k=5) == -2              # k > vocab
    assert head(T=-0.1) == -2
    assert head(T=float("nan")) == -2
    assert head(h=None) == -1
    assert head(idx=None) == -1
    assert head(seeds=None) == -1            # a sampled draft needs seeds
    assert head(seeds=None, draft=None) == -4  # no draft: no seeds needed; fails on workspace only
    assert head(seeds=None, T=0.0) == -4
    assert head(k=17) == -3
    assert head(d=5100) == -3
    assert head(w=ctypes.c_void_p(0x1008)) == -3
    assert head() == -4
    assert dfl.dflash_lm_head_topk_workspace_size(256, 5120, 151936, 8) > 0
    assert dfl.dflash_lm_head_topk_workspace_size(0, 5120, 151936, 8) == 0


def test_lm_head_vocab_limit():
    assert head(V=1048577) == -3


def test_lm_head_d_model_limit():
    assert head(d=65536 + 64) == -3


def topp(**kw):
    a = dict(z=P, out=P, kept=None, rows=4, V=151936, T=0.7, p=0.99, st=None)
    a.update(kw)
    return dfl.load().dflash_top_p_mask(a["z"], a["out"], a["kept"], a["rows"], a["V"], a["T"],
                                        a["p"], a["st"])


def test_top_p_validation():
    assert topp(rows=0) == 0
    assert topp(rows=-1) == -2
    assert topp(V=0) == -2
    assert topp(T=0.0) == -2
    assert topp(T=float("inf")) == -2
    assert topp(p=0.0) == -2
    assert topp(p=1.5) == -2
    assert topp(p=float("nan")) == -2
    assert topp(z=None) == -1
    assert topp(out=None) == -1


def topcut(**kw):
    a = dict(z=P, cut=P, kept=None, rows=4, V=151936, T=0.7, p=0.99, st=None)
    a.update(kw)
    return dfl.load().dflash_top_p_cut(a["z"], a["cut"], a["kept"], a["rows"], a["V"], a["T"],
                                       a["p"], a["st"])


def test_top_p_cut_validation():
    assert topcut(rows=0) == 0
    assert topcut(rows=-1) == -2
    assert topcut(T=0.0) == -2
    assert topcut(p=1.5) == -2
    assert topcut(p=0.0, cut=None) == -2      # shape before pointers
    assert topcut(z=None) == -1
    assert topcut(cut=None) == -1
    assert topcut(V=1 << 24) == -3
    assert topcut(rows=(1 << 20) + 1) == -3
    assert topp(out=None, kept=P) == -1       # the mask entry still needs its rows


def test_top_p_vocab_limit():
    """Fixed-point row sums (2^40 per maximal weight) stay within 64 bits only
    below 2^24 entries."""
    assert topp(V=(1 << 24)) == -3
    assert topp(V=(1 << 24) + 4) == -3


def _verify_inputs(B=2, G=4, V=64):
    import torch
    return (torch.zeros((B, G, V), dtype=torch.float32), torch.zeros((B, G, V), dtype=torch.float32),
            torch.zeros((B, G), dtype=torch.int32), torch.zeros(B, dtype=torch.int64))


@pytest.mark.parametrize("name,bad", [
    ("accept_len", ("int64", (2,))),        # wrong dtype: the kernel writes int32
    ("accept_len", ("int32", (3,))),
    ("out_tokens", ("int32", (2, 3))),      # [B, G-1] instead of [B, G]: writes past the end
    ("out_tokens", ("int64", (2, 4))),
    ("accepted", ("uint8", (2, 2))),        # [B, G-2]
    ("accepted", ("int32", (2, 3))),
])
def test_spec_verify_binding_checks_caller_outputs(name, bad):
    """Caller-supplied outputs are checked (dtype, shape, device) before the
    library is called: a wrong one would let the kernels write past it."""
    import torch
    zp, zq, d, seeds = _verify_inputs()
    dtype, shape = bad
    out = {name: torch.zeros(shape, dtype=getattr(torch, dtype))}
    with pytest.raises((TypeError, ValueError)):
        dfl.spec_verify(zp, zq, d, 0.7, seeds=seeds, outputs=out)


def test_binding_checks_workspace_dtype_and_device():
    import torch
    zp, zq, d, seeds = _verify_inputs()
    with pytest.raises(TypeError):
        dfl.spec_verify(zp, zq, d, 0.7, seeds=seeds,
                        workspace=torch.zeros(1 << 20, dtype=torch.float32))
    with pytest.raises(ValueError):
        dfl.spec_verify(zp, zq, d, 0.7, seeds=seeds,
                        workspace=torch.empty(1 << 20, dtype=torch.uint8, device="meta"))
    with pytest.raises(TypeError):
        dfl.dflash_topk(zq, 4, 0.7, seeds=seeds,
                        workspace=torch.zeros(1 << 20, dtype=torch.int32))


def verify_na(**kw):
    a = dict(zp=P, zq=P, d=P, lse=None, tc=None, dc=None, T=0.7, seeds=P, step=0, j=P, out=P,
             acc=None, B=2, G=8, V=151936, st=None)
    a.update(kw)
    return dfl.load().spec_verify_noalloc(a["zp"], a["zq"], a["d"], a["lse"], a["tc"], a["dc"], a["T"],
                                          a["seeds"],
                                          a["step"], a["j"], a["out"], a["acc"], a["B"], a["G"],
                                          a["V"], a["st"])


def test_verify_noalloc_validation_before_any_hip_call():
    """Same checks as spec_verify, then the static scratch's limit, all before
    the first HIP call (no GPU here)."""
    assert verify_na(B=0) == 0
    assert verify_na(zp=None) == -1
    assert verify_na(seeds=None) == -1
    assert verify_na(G=0) == -2
    assert verify_na(T=-1.0) == -2
    assert verify_na(G=33) == -3
    assert verify_na(V=1001) == -3
    cap = dfl.spec_verify_noalloc_max_scratch()
    assert cap == 8 << 20
    assert dfl.spec_verify_workspace_size(1024, 32, 151936) > cap
    assert verify_na(B=1024, G=32) == -6
    assert dfl.dflash_status_string(-6) != "unknown status"


M31 = 2**31 - 1


def test_workspace_queries_at_extreme_sizes():
    """Shapes an entry point rejects get 0 from its query, computed without any
    overflowing intermediate (the sanitizer build of this file turns one into
    a failure); an empty batch needs no workspace."""
    assert dfl.dflash_block_attn_workspace_size(0, 8, 40, 8, 128, 4096) == 0
    assert dfl.dflash_block_attn_workspace_size(M31, 8, 40, 8, 128, 4096) == 0
    assert dfl.dflash_block_attn_workspace_size(1, 8, 40, 8, 128, M31 - 63) == 0
    assert dfl.dflash_block_attn_workspace_size(1, 8, M31, 1, 128, 4096) == 0
    assert dfl.spec_verify_workspace_size(M31, M31, M31) == 0
    assert dfl.spec_verify_workspace_size(M31, 8, 151936) == 0
    assert dfl.spec_verify_workspace_size(1 << 17, 8, 151936) > 0   # 2^20 rows: the cap
    assert dfl.spec_verify_workspace_size((1 << 17) + 1, 8, 151936) == 0
    assert dfl.dflash_context_fuse_workspace_size(M31, 5, 5120, 5120, 5, 8, 128) == 0
    assert dfl.dflash_context_fuse_workspace_size(512, M31, M31, 5120, 5, 8, 128) == 0
    assert dfl.dflash_context_fuse_workspace_size(512, 5, 5120, 5120, M31, M31, M31) == 0
    assert dfl.dflash_lm_head_topk_workspace_size(M31, 5120, 151936, 8) == 0
    assert dfl.dflash_lm_head_topk_workspace_size(256, 5120, M31, 8) == 0
    assert dfl.dflash_lm_head_topk_workspace_size(256, M31, 151936, 8) == 0


def test_entry_points_reject_extreme_sizes():
    """Sizes whose derived counts (rows, products of heads and positions,
    launch extents) would leave 32 bits are unsupported, not wrapped."""
    assert attn(B=M31) == -3
    assert attn(W=(1 << 28) + 64) == -3
    assert attn(W=M31) == -3
    assert topk(B=M31) == -3
    assert topk(B=(1 << 17) + 1) == -3
    assert verify(B=M31) == -3
    assert verify_na(B=M31) == -3
    assert select(B=M31) == -3
    assert select(G=M31) == -3
    assert conv(B=M31) == -3
    assert conv(B=M31, G=M31) == -3
    assert fuse(rows=65536) == -3
    assert fuse(taps=M31, dt=M31) == -3
    assert fuse(nl=M31, nkv=M31, dh=M31) == -3
    assert head(rows=M31) == -3
    assert head(rows=(1 << 20) + 1) == -3
    assert topp(rows=(1 << 20) + 1) == -3


def test_device_checks_entry_points():
    """The release library records nothing (dflash_violations is unsupported
    and makes no HIP call); the build with device checks says so, exports the
    same entry points, and rejects a NULL word before any HIP call."""
    lib = dfl.load()
    assert lib.dflash_device_checks() == 0
    word = ctypes.c_uint32(7)
    assert lib.dflash_violations(ctypes.byref(word), 1, None) == -3 and word.value == 0
    assert lib.dflash_violations(None, 1, None) == -1
    checked = ctypes.CDLL(dfl.checked_lib_path)
    for n in declared_functions():
        assert hasattr(checked, n), n
    checked.dflash_device_checks.restype = ctypes.c_int
    checked.dflash_violations.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert checked.dflash_device_checks() == 1
    assert checked.dflash_violations(None, 1, None) == -1
