"""The ABI layer's host code (argument checks, error messages, launch policy
up to the first HIP call) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only, and driven by the CPU ABI
tests in a child process with clang's ASan runtime preloaded: they pass
without a sanitizer report.  The kernels are the objects build() made."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_block_paged_amd")
KERNEL_OBJS = [os.path.join(PKG, "_build", f + ".o")
               for f in ("decode_score.hip", "prefill_score.hip", "topk.hip")]
# host-side sanitizers only: each flag right after -Xarch_host
SAN_COMPILE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()
SAN_LINK = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -shared-libsan".split()


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


CHILD = """
import sys
sys.path.insert(0, ROOT)
import sparse_attention_block_paged_amd._binding as B
B.LIB_PATH = LIB
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", TESTS]))
"""


@pytest.mark.skipif(_runtime() is None, reason="clang's ASan runtime is not installed")
def test_abi_layer_under_asan_ubsan(tmp_path):
    from sparse_attention_block_paged_amd import build as hb
    if not all(os.path.exists(o) for o in KERNEL_OBJS):
        pytest.skip("the kernel objects are built by __graft_entry__.build()")
    cc = hb.hipcc()
    obj, lib = str(tmp_path / "abi.o"), str(tmp_path / "libmm3idx_san.so")
    subprocess.check_call([cc, "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={hb.ARCH}",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN_COMPILE,
                           "-I", hb.INCLUDE, "-I", hb.CSRC, "-c", os.path.join(hb.CSRC, "mm3_abi.hip"),
                           "-o", obj], stderr=subprocess.DEVNULL)
    subprocess.check_call([cc, f"--offload-arch={hb.ARCH}", "-shared", "-fPIC", *SAN_LINK, "-o", lib, obj,
                           *KERNEL_OBJS], stderr=subprocess.DEVNULL)
    code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\nTESTS = {os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}\n" + CHILD
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
