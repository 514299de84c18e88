"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code): small cases of every entry point -- uniform bf16 and NVFP4
decode, a ragged batch with prefix lengths and an empty request, the sparse
block table -- run without a sanitizer report and give byte-identical
results to the normal build.  The child process uses numpy only."""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent("""
    import hashlib, sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    oracle._LIB = LIB  # newer than its source, so it is loaded as it is
    rng = np.random.default_rng(7)
    h = hashlib.sha256()

    def bf16(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    def table(lens, width):
        n = sum(-(-l // 128) for l in lens)
        perm = rng.permutation(n).astype(np.int32)
        bt = np.full((len(lens), width), n, dtype=np.int32)  # unused: one spare page
        at = 0
        for r, l in enumerate(lens):
            k = -(-l // 128)
            bt[r, :k] = perm[at:at + k]
            at += k
        return bt, n + 1

    H, Q, W = 2, 4, 16
    lens = np.array([1000, 130, 4], dtype=np.int32)
    bt, pages = table(lens, W)
    q = bf16((lens.size * Q, H, 128))
    kd = bf16((pages, 128, 128))
    s, ids = oracle.forward(q, 0, kd, None, bt, lens, Q, 0.0884, 4, 1, 1, W)
    h.update(s.tobytes()); h.update(ids.tobytes())
    s_b, s64, ids_b = oracle.forward(q, 0, kd, None, bt, lens, Q, 0.0884, 4, 1, 1, W, with64=True)
    h.update(s_b.tobytes()); h.update(s64.tobytes()); h.update(ids_b.tobytes())

    nib = rng.integers(0, 256, (pages, 128, 64), dtype=np.uint8)
    sc = rng.integers(0x20, 0x50, (pages, 128, 8), dtype=np.uint8)
    s4, ids4 = oracle.forward(q, 1, nib, sc, bt, lens, Q, 0.0884, 4, 1, 1, W)
    h.update(s4.tobytes()); h.update(ids4.tobytes())

    rlens = np.array([1000, 130, 130], dtype=np.int32)
    rbt, rpages = table(rlens, W)
    cu = np.array([0, 3, 3, 7], dtype=np.int32)
    pre = np.array([990, 0, 120], dtype=np.int32)
    rq = bf16((7, H, 128))
    rk = bf16((rpages, 128, 128))
    sr, idr = oracle.forward(rq, 0, rk, None, rbt, rlens, 4, 0.0884, 4, 1, 1, W,
                             cu_seqlens_q=cu, prefix_lens=pre)
    h.update(sr.tobytes()); h.update(idr.tobytes())

    P = 2
    abt = rng.integers(0, 1000, (lens.size, W * P), dtype=np.int32)
    st, ctx = oracle.sparse_block_table(ids[0], lens, Q, abt, P, P)
    h.update(st.tobytes()); h.update(ctx.tobytes())
    print(h.hexdigest())
""")


def _asan_runtime():
    if shutil.which("gcc") is None:
        return None
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _run(lib, env):
    code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + CHILD
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          env=env, timeout=300)


@pytest.mark.skipif(_asan_runtime() is None, reason="gcc with libasan is not available")
def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    src = os.path.join(ROOT, "oracle", "mm3_oracle.c")
    san = str(tmp_path / "libmm3oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-fast-math", "-ffp-contract=off", "-o", san, src, "-lm"])
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run(san, env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    plain = _run(oracle.build(force=False), dict(os.environ))
    assert plain.returncode == 0, plain.stderr[-4000:]
    assert r.stdout.strip() == plain.stdout.strip() and len(r.stdout.strip()) == 64
