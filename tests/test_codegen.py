"""Code-generation invariants of the gfx950 kernels, checked on the host.

Every kernel addresses global memory with global_* instructions and LDS with
ds_* instructions whose address space is known at compile time: no generic
(flat_*) addressing, no private-segment (scratch_*) traffic and no device
function calls.  The device assembly is produced by hipcc from the library's
own sources (nothing prebuilt is read)."""
import os
import re
import subprocess

import pytest

from block_drafting_context_amd import build as b

SOURCES = [s for s in b.SOURCES if s.endswith(".hip")]


def device_asm(src, checked=False):
    """Device assembly of one source, as the release library or (checked) as
    the library built with device-data checks compiles it."""
    extra = b.CHECKED_FLAGS if checked else []
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O3",
           "-std=c++17", "-S", "--cuda-device-only", *b.DEVICE_FLAGS, *extra, f"-I{b.INCLUDE}",
           f"-I{b.CSRC}", os.path.join(b.CSRC, src), "-o", "-"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stdout


@pytest.mark.parametrize("checked", [False, True], ids=["release", "checked"])
@pytest.mark.parametrize("src", SOURCES)
def test_no_generic_or_private_addressing(src, checked):
    asm = device_asm(src, checked)
    bad = {}
    fn = None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn = m.group(1)
        ins = line.strip().split(" ")[0]
        if ins.startswith(("flat_", "scratch_", "s_swappc")):
            bad.setdefault(fn, set()).add(ins)
    assert not bad, f"{src}: {bad}"


def test_lm_head_m0_is_written_only_for_its_lds_dma():
    """The LM head's LDS DMA is inline assembly that sets m0 (the LDS
    destination) itself.  Nothing else in that file may read or write m0, so
    no compiler-held value there can be overwritten: every m0 write is
    followed by one wait state (an LDS DMA must not read m0 in the instruction
    right after a scalar write of it) and then by the DMA that reads it."""
    lines = [l.strip() for l in device_asm("lm_head.hip").splitlines()]
    ins = [l for l in lines if l and not l.startswith((";", ".", "_")) and not l.endswith(":")]
    writes = 0
    for i, l in enumerate(ins):
        if "m0" not in l.split(";")[0]:
            continue
        op = l.split()[0]
        if op == "s_mov_b32" and l.split()[1].rstrip(",") == "m0":
            writes += 1
            assert i + 2 < len(ins) and ins[i + 1] == "s_nop 0", ins[i + 1]
            assert re.match(r"buffer_load_dwordx4 .* lds", ins[i + 2]), ins[i + 2]
        else:
            raise AssertionError(f"unexpected m0 use: {l}")
    assert writes > 0
