"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer run of the C ABI.

The library's host code (argument checks, the decode plan, workspace sizes,
launch set-up) is compiled with ``-fsanitize=address,undefined`` and driven by
``tests/sanitize/abi_fuzz.c``: every entry point with edge-value integers,
non-finite floats, NULL and misaligned pointers.  Any memory error or
undefined behaviour (signed overflow, an enum value out of range, ...) aborts
the run.  Device code is compiled unoptimised only so that the objects link;
it never runs: the driver exits without calling anything when a GPU is
visible, and this test is skipped there.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_qk_online_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_fuzz.c")
OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/llvm/bin"
KERNELS = ["decode.hip", "prefill.hip", "prefill256.hip", "merge.hip"]
HEADERS = [os.path.join(CSRC, h) for h in ("common.h", "launch.h")] + [os.path.join(INCLUDE, "attn.h")]
# Host code only: each -fsanitize= applies to the host compilation.
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]


def _digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def _object(src, cmd_tail):
    """Compile `src` unless an object built from the same sources exists."""
    tag = _digest([os.path.join(CSRC, src)] + HEADERS)
    obj = os.path.join(OUT, f"{os.path.splitext(src)[0]}-{tag}.o")
    if not os.path.exists(obj):
        stem = os.path.splitext(src)[0] + "-"
        for old in os.listdir(OUT):
            if old.startswith(stem) and old.endswith(".o"):
                os.remove(os.path.join(OUT, old))
        _run(cmd_tail + ["-c", os.path.join(CSRC, src), "-o", obj + ".tmp"])
        os.replace(obj + ".tmp", obj)
    return obj


def _build():
    os.makedirs(OUT, exist_ok=True)
    cxx = os.path.join(LLVM, "clang++")
    inc = ["-I", INCLUDE, "-I", CSRC]
    host = ["-Xarch_host", "-O1", "-Xarch_host", "-g", "-fno-omit-frame-pointer"]
    kernel_cmd = [cxx, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", *host,
                  "-Xarch_device", "-O0", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                  *SAN, *inc, "-w"]
    api_cmd = [cxx, "-x", "hip", "--offload-host-only", "-std=c++17", *host, "-Wall", "-Werror",
               *SAN, *inc]
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _object(s, kernel_cmd), KERNELS))
    objs.append(_object("api.cpp", api_cmd))
    drv = os.path.join(OUT, "abi_fuzz.o")
    _run([os.path.join(LLVM, "clang"), "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *SAN,
          "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", INCLUDE, "-c", DRIVER, "-o", drv])
    exe = os.path.join(OUT, "abi_fuzz")
    _run([cxx, "-Xarch_host", "-fsanitize=address,undefined", "-o", exe, drv, *objs,
          "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    return exe


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host-only fuzz with fake device "
                    "pointers: runs where no GPU is present")
@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "clang++")),
                    reason="ROCm clang not installed")
def test_abi_fuzz_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=600)
    if r.returncode == 77:
        pytest.skip(r.stdout.strip())
    assert r.returncode == 0, f"rc={r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert " 0 failures" in r.stdout, r.stdout
    # Every base configuration reached the launch (ATTN_E_HIP without a GPU).
    assert "HIP runtime error=0" not in r.stdout, r.stdout
