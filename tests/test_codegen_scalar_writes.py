"""Code-generation invariant of the gfx950 kernels, checked on the host: no
kernel writes memory through the scalar data cache.  Every store and atomic
is a vector-memory (global_*, buffer_*, ds_*) instruction; the scalar unit only
reads (kernel arguments, uniform loads).  The device assembly is produced by
hipcc from the library's own sources."""
import re

import pytest

from test_codegen import SOURCES, device_asm

SCALAR_WRITES = re.compile(r"^s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")


@pytest.mark.parametrize("checked", [False, True], ids=["release", "checked"])
@pytest.mark.parametrize("src", SOURCES)
def test_no_scalar_memory_writes(src, checked):
    bad = {}
    fn = None
    for line in device_asm(src, checked).splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            fn = m.group(1)
        ins = line.strip().split(" ")[0]
        if SCALAR_WRITES.match(ins):
            bad.setdefault(fn, set()).add(ins)
    assert not bad, f"{src}: {bad}"
