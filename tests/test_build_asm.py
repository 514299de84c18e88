"""Properties of the gfx950 code that the sources rely on, checked in the
compiler's assembly (CPU only: hipcc cross-compiles).

prefill_score.hip moves its key pages into LDS with global_load_lds_dwordx4
issued from inline assembly that sets M0 itself; that is only sound while no
compiler-generated instruction of the file reads M0.  And the scorers' hot
loops must not spill to scratch."""
import os
import re
import shutil
import subprocess

import pytest

from sparse_attention_block_paged_amd import build as B


def _asm(tmp_path, src):
    out = str(tmp_path / (src + ".s"))
    cmd = [B.hipcc(), *B.HIP_FLAGS, *B.SOURCE_FLAGS.get(src, []), "-I", B.INCLUDE, "-I", B.CSRC,
           "-S", "--cuda-device-only", os.path.join(B.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def _kernels(asm):
    """{symbol: [instruction lines]} for every kernel in the file."""
    out, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1)
            out[cur] = []
        elif cur is not None:
            t = line.split(";")[0].strip()
            if t and not t.startswith("."):
                out[cur].append(t)
                if t == "s_endpgm":
                    cur = None
    return out


def _scratch(asm):
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"^(_Z\w+):.*?; ScratchSize: (\d+)", asm, re.S | re.M)}


pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def test_prefill_m0_only_set_by_the_page_copies(tmp_path):
    kernels = _kernels(_asm(tmp_path, "prefill_score.hip"))
    assert any("prefill_score_kernel" in k for k in kernels)
    for name, ins in kernels.items():
        for i, t in enumerate(ins):
            if "m0" not in t:
                continue
            # the page copy: s_mov_b32 m0, sN; s_nop 0; global_load_lds_dwordx4
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", t), f"{name}: compiler code uses M0: {t}"
            assert ins[i + 1] == "s_nop 0" and ins[i + 2].startswith("global_load_lds_dwordx4"), (
                f"{name}: M0 set outside a page copy: {ins[i:i + 3]}")


def test_scorer_multiply_loops_do_not_spill(tmp_path):
    """Decode scorers and the prefill scorers without the fused selection use
    no scratch at all; the fused prefill scorers may spill only outside the
    loop that issues the multiplies (none of their spill accesses sits
    between the first and last MFMA)."""
    for src in ("decode_score.hip", "prefill_score.hip"):
        asm = _asm(tmp_path, src)
        sizes = _scratch(asm)
        kernels = _kernels(asm)
        for name, size in sizes.items():
            if size == 0:
                continue
            assert "prefill_score_kernel" in name and not name.split("Lb")[1].split("ELi")[1].startswith("0"), (
                f"{name} spills {size} bytes")
            ins = kernels[name]
            mf = [i for i, t in enumerate(ins) if t.startswith("v_mfma")]
            sc = [i for i, t in enumerate(ins) if t.startswith("scratch_")]
            assert all(i < mf[0] or i > mf[-1] for i in sc), f"{name}: scratch access inside the MFMA loop"
