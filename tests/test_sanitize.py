"""Host sanitizers over the C ABI's host code: the library is rebuilt with
AddressSanitizer and UndefinedBehaviorSanitizer on its host side only (device
code is compiled as usual), linked into the driver ``tests/native/abi_checks.cpp``,
and run.  Without a GPU the driver exercises every argument and state check
that precedes a device call; with a GPU present the same binary also drives a small
cache end to end (create, prefill, decode, read, statistics, destroy)."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_eviction_prefill_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "native", "abi_checks.cpp")
OUT = os.path.join(ROOT, "kv_cache_eviction_prefill_amd", "_build", "sanitize")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tool(name):
    for cand in (shutil.which(name), f"/opt/rocm/bin/{name}", f"/opt/rocm/lib/llvm/bin/{name}"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip(f"{name} not found")


def _build():
    from kv_cache_eviction_prefill_amd import build as b

    os.makedirs(OUT, exist_ok=True)
    hipcc = _tool("hipcc")
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        procs.append(subprocess.Popen([hipcc, *b.COMMON, "-g", *HOST_SAN, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    drv = os.path.join(OUT, "abi_checks.o")
    procs.append(subprocess.Popen([hipcc, "-O1", "-g", "-std=c++17", "-I", b.INCLUDE, *HOST_SAN, "-c", DRIVER,
                                   "-o", drv], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    exe = os.path.join(OUT, "abi_checks")
    # the link names no HIP source: the sanitizer runtimes come in on the host link only
    link = [_tool("clang++"), "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    res = subprocess.run(link, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


def _run(exe):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-4000:]
    assert "abi checks ok" in res.stdout, text[-4000:]
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-4000:]
    return res.stdout.strip()


@pytest.mark.slow
def test_abi_checks_under_host_sanitizers():
    print(_run(_build()))


@pytest.mark.gpu
def test_abi_end_to_end_under_host_sanitizers():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    out = _run(_build())
    assert "end-to-end" in out, out
