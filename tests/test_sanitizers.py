"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds are made in a temporary folder and exercised in child processes:
  * oracle.c, compiled by gcc with both sanitizers, runs the oracle's own pin
    tests (tests/test_oracle_*.py);
  * libdflash.so from the same sources as the product build, with the
    sanitizers applied to the host pass only (argument checks, workspace
    queries, layout arithmetic; the device code is unchanged), runs the C-ABI
    tests (tests/test_abi.py), which call every entry point with rejected
    arguments and extreme sizes.  No kernel is launched.
Each child preloads the matching runtime (gcc's libasan and libubsan; clang's
asan runtime, which also carries the UBSan handlers) and a report aborts it.
Before trusting a clean run, a planted heap overflow and a planted signed
overflow in a small library loaded the same way must be reported.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

from block_drafting_context_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-g"]

PLANTED = r"""
#include <stdlib.h>
int heap_overflow(int n) { int* p = (int*)malloc(n * sizeof(int)); int v = p[n]; free(p); return v; }
int signed_overflow(int a) { return a + 1; }
"""


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res


def _file_name(compiler, name):
    path = _run([compiler, f"-print-file-name={name}"]).stdout.strip()
    assert os.path.isabs(path) and os.path.exists(path), (compiler, name, path)
    return path


@pytest.fixture(scope="module")
def runtimes():
    return {"gcc": ":".join(_file_name("gcc", n) for n in ("libasan.so", "libubsan.so")),
            "clang": _file_name(CLANG, "libclang_rt.asan-x86_64.so")}


def _child_env(preload, **extra):
    env = dict(os.environ)
    env.update(LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1", **extra)
    return env


def _python(code, env):
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                          cwd=ROOT, timeout=600)


@pytest.mark.parametrize("kind", ["gcc", "clang"])
def test_planted_errors_are_reported(tmp_path, runtimes, kind):
    src = tmp_path / "planted.c"
    src.write_text(PLANTED)
    lib = tmp_path / f"planted_{kind}.so"
    if kind == "gcc":
        _run(["gcc", "-O0", *GCC_SAN, "-fPIC", "-shared", "-o", str(lib), str(src)])
    else:
        _run([CLANG, "-O0", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-shared-libsan", "-fPIC", "-shared", "-o", str(lib), str(src)])
    env = _child_env(runtimes[kind])
    load = f"import ctypes; lib = ctypes.CDLL({str(lib)!r}); "
    heap = _python(load + "lib.heap_overflow(7)", env)
    assert heap.returncode != 0 and "heap-buffer-overflow" in heap.stderr, heap.stderr[-2000:]
    sig = _python(load + "lib.signed_overflow(2**31 - 1)", env)
    assert sig.returncode != 0 and "signed integer overflow" in sig.stderr, sig.stderr[-2000:]
    ok = _python(load + "print(lib.signed_overflow(5))", env)
    assert ok.returncode == 0 and ok.stdout.strip() == "6", ok.stderr[-2000:]


@pytest.fixture(scope="module")
def oracle_san(tmp_path_factory):
    out = tmp_path_factory.mktemp("oracle_san") / "liboracle_san.so"
    _run(["gcc", "-O1", *GCC_SAN, "-fopenmp", "-fPIC", "-shared", "-std=gnu11", "-o", str(out),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    return str(out)


@pytest.fixture(scope="module")
def lib_san(tmp_path_factory):
    """libdflash.so from the product's sources and flags, host pass sanitized;
    one hipcc process per source, then a plain link (the sanitizer symbols
    resolve against the preloaded runtime)."""
    d = tmp_path_factory.mktemp("lib_san")
    flags = [f for f in libbuild.FLAGS if f != "-shared"]
    objs = [str(d / (os.path.splitext(s)[0] + ".o")) for s in libbuild.SOURCES]

    def compile_one(src_obj):
        src, obj = src_obj
        _run([HIPCC, *flags, *HOST_SAN, "-c", os.path.join(libbuild.CSRC, src), "-o", obj])

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(compile_one, zip(libbuild.SOURCES, objs)))
    out = str(d / "libdflash_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out])
    syms = _run(["nm", "-D", out]).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms  # both passes instrumented
    return out


def test_oracle_pins_under_sanitizers(runtimes, oracle_san):
    env = _child_env(runtimes["gcc"], DFLASH_ORACLE_LIB=oracle_san)
    code = ("import sys, pytest, oracle; lib = oracle._load(); "
            f"assert lib._name == {oracle_san!r}, lib._name; "
            f"sys.exit(pytest.main(['-q', '-x', '--capture=sys', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            f"*sorted(__import__('glob').glob({TESTS!r} + '/test_oracle_*.py'))]))")
    res = _python(code, env)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout and "failed" not in res.stdout


def test_host_checks_under_sanitizers(runtimes, lib_san):
    env = _child_env(runtimes["clang"], DFLASH_LIB=lib_san)
    code = ("import sys, pytest, block_drafting_context_amd as dfl; lib = dfl.load(); "
            f"assert lib._name == {lib_san!r}, lib._name; "
            f"sys.exit(pytest.main(['-q', '-x', '--capture=sys', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            f"{os.path.join(TESTS, 'test_abi.py')!r}]))")
    res = _python(code, env)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout and "failed" not in res.stdout
