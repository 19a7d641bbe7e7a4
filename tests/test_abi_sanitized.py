"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

abi.hip (argument validation, workspace sizing, grid sizing, status codes) is compiled with the
sanitizers on its host side only (device code is unchanged), linked with the other objects of the
regular build (_build/, written by __graft_entry__.build()), and tests/test_abi_host.py is run
against that library in a child process with the sanitizer runtime preloaded.  Any report ends the
child with a nonzero status."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gqa_paged_kv_attention_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
# host-side sanitizers only: each -fsanitize= follows -Xarch_host
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all".split()


def _others():
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    return [o for o in objs if not os.path.basename(o).startswith("abi.")]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs ROCm's hipcc and clang")
def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    others = _others()
    if len(others) < 5:
        pytest.skip("regular build objects missing (run __graft_entry__.build())")
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("AddressSanitizer runtime not found")
    obj, lib = str(tmp_path / "abi_san.o"), str(tmp_path / "libgqa_paged_san.so")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    r = subprocess.run([HIPCC] + flags + SAN + ["-c", os.path.join(CSRC, "abi.hip"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-shared-libasan"] + SAN[:4] +
                       ["-o", lib, obj] + others, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, GQA_TEST_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "passed" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
