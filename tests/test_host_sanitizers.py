"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library sources are compiled with the sanitizers on the host side only
(device code is built as usual and never run), linked with the argument
fuzzer tests/sanitize/abi_fuzz.cpp, and run on the CPU: every entry point and
the workspace sizing are called with edge-value shapes, strides, pointers and
workspaces.  Any sanitizer report fails the test.  Skipped where a GPU is
visible (the fuzzer passes fake device pointers, and refuses to run there
too)."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "free_block_sparse_major_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-g"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-fPIC", "-std=c++20", "-I" + os.path.join(ROOT, "include"),
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.skipif(_gpu_visible(), reason="runs on hosts without a GPU only")
def test_abi_fuzz_under_sanitizers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = [(os.path.join(CSRC, s), str(tmp_path / (s[:-4] + ".o")), ()) for s in srcs]
    jobs.append((os.path.join(ROOT, "tests", "sanitize", "abi_fuzz.cpp"),
                 str(tmp_path / "abi_fuzz.o"), ("-x", "hip")))

    def compile_one(job):
        src, obj, extra = job
        r = subprocess.run([HIPCC, *FLAGS, *SAN, *extra, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        return src, r

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        for src, r in ex.map(compile_one, jobs):
            assert r.returncode == 0, (src, r.stderr[-3000:])
    exe = str(tmp_path / "abi_fuzz")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *[j[1] for j in jobs], "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "calls by status" in out
    shutil.rmtree(tmp_path, ignore_errors=True)
