"""The C ABI without a GPU: exports, struct layout, host-side validation.

Validation happens before anything is enqueued, so these calls use fake
(never dereferenced) device pointers and run on a machine with no GPU.  Each
rejected call must return its documented code and describe the problem.
"""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_block_paged_amd as mm3
from sparse_attention_block_paged_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mm3_index.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(mm3_\w+)\s*\(", txt, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 7
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTED)
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, re.M), f"{n} not a defined text symbol"


@pytest.mark.parametrize("cname,cls", [("mm3_problem", B.Problem), ("mm3_rows", B.Rows),
                                       ("mm3_sparse_out", B.SparseOut)])
def test_struct_layout_matches_header(tmp_path, cname, cls):
    src = tmp_path / "layout.c"
    fields = [f[0] for f in cls._fields_]
    body = "".join(f'printf("%zu ", offsetof({cname}, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "mm3_index.h"\n'
                   f'int main(void){{ {body} printf("%zu\\n", sizeof({cname})); return 0; }}\n')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    want = [getattr(cls, f).offset for f in fields] + [ctypes.sizeof(cls)]
    assert got == want


FAKE = 1 << 20  # 16-byte aligned, never dereferenced


ROW_FIELDS = {f[0] for f in B.Rows._fields_}


def _rows(**kw):
    m = B.Rows()
    d = dict(seq_lens=FAKE * 4, cu_seqlens_q=None, prefix_lens=None, num_reqs=8, query_len=4,
             total_q=None, max_seq_len=8192)
    d.update(kw)
    if d["total_q"] is None:
        d["total_q"] = d["num_reqs"] * d["query_len"]
    for k, v in d.items():
        setattr(m, k, v)
    return m


def _problem(**kw):
    p = B.Problem()
    d = dict(q=FAKE, q_tok_stride=4 * 128, q_head_stride=128, heads=4, kfmt=0, kdata=FAKE * 2,
             kscales=None, num_pages=100, block_table=FAKE * 3, bt_row_stride=64, bt_width=64,
             sm_scale=0.088)
    rk = {k: v for k, v in kw.items() if k in ROW_FIELDS}
    d.update({k: v for k, v in kw.items() if k not in ROW_FIELDS})
    for k, v in d.items():
        setattr(p, k, v)
    p.rows = _rows(**rk)
    return p


def _score(p, sh=None, sr=64, sw=64, scores=FAKE * 5):
    T = p.rows.total_q
    sh = T * sr if sh is None else sh
    return B.lib().mm3_index_score(ctypes.byref(p), scores, sh, sr, sw, None)


def _err():
    return B.lib().mm3_last_error().decode()


BAD_PROBLEMS = [
    ("heads", dict(heads=0), "heads"),
    ("query_len", dict(query_len=0), "query_len"),
    ("num_reqs", dict(num_reqs=-1), "num_reqs"),
    ("max_seq_len", dict(max_seq_len=-5), "max_seq_len"),
    ("too_many_blocks", dict(max_seq_len=65535 * 128, bt_width=70000, bt_row_stride=70000), "65535"),
    ("sm_scale_zero", dict(sm_scale=0.0), "sm_scale"),
    ("sm_scale_neg", dict(sm_scale=-1.0), "sm_scale"),
    ("sm_scale_nan", dict(sm_scale=float("nan")), "sm_scale"),
    ("sm_scale_inf", dict(sm_scale=float("inf")), "sm_scale"),
    ("kfmt", dict(kfmt=7), "format"),
    ("no_pages", dict(num_pages=0), "page"),
    ("null_q", dict(q=None), "non-NULL"),
    ("null_table", dict(block_table=None), "non-NULL"),
    ("null_lens", dict(seq_lens=None), "seq_lens"),
    ("nvfp4_no_scales", dict(kfmt=1), "kscales"),
    ("q_misaligned", dict(q=FAKE + 8), "aligned"),
    ("k_misaligned", dict(kdata=FAKE * 2 + 4), "aligned"),
    ("q_stride", dict(q_tok_stride=4 * 128 + 4), "multiples of 8"),
    ("q_head_overlap", dict(q_head_stride=64), "head stride"),
    ("table_narrow", dict(bt_width=63), "narrower"),
    ("table_row_stride", dict(bt_row_stride=32), "row stride"),
    ("tokens_overflow", dict(num_reqs=1 << 20, query_len=1 << 12, total_q=0), "total_q"),
    ("rows_overflow", dict(heads=1 << 16, query_len=1 << 16, q_head_stride=128), "2^31"),
    ("total_q_mismatch", dict(total_q=31), "total_q"),
    ("total_q_negative", dict(cu_seqlens_q=FAKE * 8, total_q=-1), "total_q"),
    ("total_q_past_grid_bound", dict(cu_seqlens_q=FAKE * 8, total_q=(1 << 31) - 1023), "2^31 - 1024"),
    ("prefix_without_cu", dict(prefix_lens=FAKE * 9), "prefix_lens needs cu_seqlens_q"),
    ("ragged_rows_without_requests", dict(cu_seqlens_q=FAKE * 8, num_reqs=0, total_q=5), "without requests"),
    ("cu_misaligned", dict(cu_seqlens_q=FAKE * 8 + 2), "aligned"),
    ("prefix_misaligned", dict(cu_seqlens_q=FAKE * 8, prefix_lens=FAKE * 9 + 1), "aligned"),
]


@pytest.mark.parametrize("label,kw,msg", BAD_PROBLEMS, ids=[b[0] for b in BAD_PROBLEMS])
def test_problem_rules(label, kw, msg):
    p = _problem(**kw)
    assert _score(p) == B.MM3_EINVAL
    assert msg in _err(), _err()
    # the same rule guards the fused entry point
    rc = B.lib().mm3_index_decode(ctypes.byref(p), 16, 1, 2, FAKE * 6, 32 * 16, 16, None, 0, 0, 0,
                                  FAKE * 7, 1 << 30, None, None)
    assert rc == B.MM3_EINVAL


BAD_SCORES = [
    ("null", dict(scores=None), "non-NULL"),
    ("misaligned", dict(scores=FAKE * 5 + 2), "aligned"),
    ("narrow", dict(sw=63), "score width"),
    ("row_stride", dict(sr=32, sw=64), "row stride"),
    ("head_stride", dict(sh=10), "head stride"),
]


@pytest.mark.parametrize("label,kw,msg", BAD_SCORES, ids=[b[0] for b in BAD_SCORES])
def test_score_buffer_rules(label, kw, msg):
    assert _score(_problem(), **kw) == B.MM3_EINVAL
    assert msg in _err(), _err()


def test_empty_batch_returns_ok_without_launch():
    assert _score(_problem(num_reqs=0)) == B.MM3_OK
    assert _err() == ""
    # ragged with no rows at all (every request empty)
    assert _score(_problem(cu_seqlens_q=FAKE * 8, total_q=0)) == B.MM3_OK
    rows = _rows(num_reqs=0)
    rc = B.lib().mm3_index_topk(FAKE, 0, 64, 64, 4, ctypes.byref(rows), 16, 1, 2, FAKE * 6, 0,
                                16, None)
    assert rc == B.MM3_OK


def test_ragged_total_q_sizes_the_buffers():
    """Ragged batches take total_q, not num_reqs * query_len, as the row count
    that score and out strides must cover."""
    p = _problem(cu_seqlens_q=FAKE * 8, prefix_lens=FAKE * 9, total_q=100, query_len=64)
    # (only rejected calls here: a valid one would launch on the fake pointers)
    assert _score(p, sh=99 * 64) == B.MM3_EINVAL and "head stride" in _err()
    rows = _rows(cu_seqlens_q=FAKE * 8, total_q=100, query_len=64)
    assert _topk(rows=rows, oh=99 * 16) == B.MM3_EINVAL and "head stride" in _err()


def _topk(**kw):
    rk = {k: kw.pop(k) for k in list(kw) if k in ROW_FIELDS}
    d = dict(scores=FAKE, sh=32 * 64, sr=64, sw=64, heads=4, topk=16, I=1, L=2, out=FAKE * 6,
             oh=32 * 16, orow=16, rows="default")
    d.update(kw)
    rows = _rows(**rk) if d["rows"] == "default" else d["rows"]
    return B.lib().mm3_index_topk(d["scores"], d["sh"], d["sr"], d["sw"], d["heads"],
                                  None if rows is None else ctypes.byref(rows), d["topk"], d["I"],
                                  d["L"], d["out"], d["oh"], d["orow"], None)


BAD_TOPK = [
    ("topk_zero", dict(topk=0), "topk"),
    ("topk_big", dict(topk=1025, orow=1025, oh=32 * 1025), "topk"),
    ("forced_exceed", dict(topk=4, I=3, L=2, orow=4, oh=128), "exceeds"),
    ("negative_init", dict(I=-1), ">= 0"),
    ("null_out", dict(out=None), "out"),
    ("out_row_stride", dict(orow=8), "row stride"),
    ("out_head_stride", dict(oh=10), "head stride"),
    ("score_width", dict(sw=10, sr=10, sh=320), "width"),
    ("null_seq", dict(seq_lens=None), "seq_lens"),
    ("null_rows", dict(rows=None), "rows"),
    ("heads", dict(heads=0), "heads"),
    ("prefix_without_cu", dict(prefix_lens=FAKE * 9), "prefix_lens"),
    ("total_q", dict(total_q=33), "total_q"),
]


@pytest.mark.parametrize("label,kw,msg", BAD_TOPK, ids=[b[0] for b in BAD_TOPK])
def test_topk_rules(label, kw, msg):
    assert _topk(**kw) == B.MM3_EINVAL
    assert msg in _err(), _err()


def test_decode_workspace_rules():
    p = _problem()
    need = B.lib().mm3_index_decode_workspace_bytes(ctypes.byref(p), 16, 0)
    assert need == 4 * 32 * 64 * 4  # heads * tokens * round_up(64, 16) * fp32
    assert B.lib().mm3_index_decode_workspace_bytes(ctypes.byref(p), 16, 1) == 0
    for ws, nbytes in [(None, need), (FAKE * 7, need - 1), (FAKE * 7 + 16, need)]:
        rc = B.lib().mm3_index_decode(ctypes.byref(p), 16, 1, 2, FAKE * 6, 32 * 16, 16, None, 0, 0,
                                      0, ws, nbytes, None, None)
        assert rc == B.MM3_EWORKSPACE, (ws, nbytes)
        assert "workspace" in _err()
    bad = _problem(heads=0)
    assert B.lib().mm3_index_decode_workspace_bytes(ctypes.byref(bad), 16, 0) == 0
    assert "heads" in _err()


def _sparse_out(abt=FAKE * 3, abt_row=128, abt_w=128, P=2, stride=2, st=FAKE * 4, st_row=32,
                ctx=FAKE * 5):
    o = B.SparseOut()
    o.attention_block_table, o.abt_row_stride, o.abt_width = abt, abt_row, abt_w
    o.pages_per_block, o.block_page_stride = P, stride
    o.sparse_table, o.st_row_stride, o.sparse_ctx_lens = st, st_row, ctx
    return o


SPARSE_KEYS = ("abt", "abt_row", "abt_w", "P", "stride", "st", "st_row", "ctx")


def _sparse(**kw):
    rk = {k: kw.pop(k) for k in list(kw) if k in ROW_FIELDS}
    sk = {k: kw.pop(k) for k in list(kw) if k in SPARSE_KEYS}
    d = dict(ids=FAKE, orow=16, topk=16)
    d.update(kw)
    rows = _rows(**rk)
    sp = _sparse_out(**sk)
    return B.lib().mm3_build_sparse_block_table(d["ids"], d["orow"], d["topk"], ctypes.byref(rows),
                                                ctypes.byref(sp), None)


BAD_SPARSE = [
    ("missing_table", dict(abt=None), "together"),
    ("missing_ctx", dict(ctx=None), "together"),
    ("stride", dict(stride=3), "block_page_stride"),
    ("narrow_abt", dict(abt_w=127, abt_row=127), "narrower"),
    ("st_row", dict(st_row=31), "sparse table row stride"),
    ("pages", dict(P=0, stride=0), "pages_per_block"),
    ("null_seq", dict(seq_lens=None), "seq_lens"),
    ("total_q", dict(total_q=5), "total_q"),
]


@pytest.mark.parametrize("label,kw,msg", BAD_SPARSE, ids=[b[0] for b in BAD_SPARSE])
def test_sparse_table_rules(label, kw, msg):
    assert _sparse(**kw) == B.MM3_EINVAL
    assert msg in _err(), _err()


def test_binding_rejects_wrong_dtypes_before_the_library():
    import torch
    q = torch.zeros((4, 1, 128), dtype=torch.float32)
    k = torch.zeros((2, 128, 128), dtype=torch.bfloat16)
    bt = torch.zeros((1, 16), dtype=torch.int32)
    sl = torch.zeros((1,), dtype=torch.int32)
    with pytest.raises(ValueError):
        mm3.make_problem(q, k, bt, sl, 4, 2048, 0.1)
    with pytest.raises(ValueError):
        mm3.make_problem(q.bfloat16(), k, bt.long(), sl, 4, 2048, 0.1)


FUSED_SPARSE_BAD = [
    ("heads", dict(), dict(), "one index head"),
    ("missing_ctx", dict(heads=1, q_head_stride=128), dict(ctx=None), "together"),
    ("stride", dict(heads=1, q_head_stride=128), dict(stride=3), "block_page_stride"),
    ("narrow_abt", dict(heads=1, q_head_stride=128), dict(abt_w=127, abt_row=127), "narrower"),
    ("st_row", dict(heads=1, q_head_stride=128), dict(st_row=31), "row stride"),
]


@pytest.mark.parametrize("label,pkw,skw,msg", FUSED_SPARSE_BAD, ids=[b[0] for b in FUSED_SPARSE_BAD])
def test_fused_sparse_table_rules(label, pkw, skw, msg):
    """The fused call's sparse-table output (page "ops.index_topk",
    minimax_m3_index_decode: arguments together, one index head, stride P or
    2P) is checked before anything is enqueued."""
    p = _problem(**pkw)
    sp = _sparse_out(**skw)
    rc = B.lib().mm3_index_decode(ctypes.byref(p), 16, 1, 2, FAKE * 6, 32 * 16, 16, None, 0, 0, 0,
                                  FAKE * 7, 1 << 30, ctypes.byref(sp), None)
    assert rc == B.MM3_EINVAL
    assert msg in _err(), _err()


def test_binding_sparse_arguments_together():
    import torch
    z = torch.zeros((4, 16), dtype=torch.int32)
    with pytest.raises(ValueError, match="together"):
        mm3.mm3_index_decode(torch.zeros((4, 1, 128), dtype=torch.bfloat16),
                             torch.zeros((2, 128, 128), dtype=torch.bfloat16), z[:1],
                             torch.zeros((1,), dtype=torch.int32), 4, 2048, 0.1, 4, 1, 1,
                             attention_block_table=z)


def _topk_blocks(**kw):
    d = dict(scores=FAKE, sh=32 * 64, sr=64, sw=64, heads=4, rb=FAKE * 4, T=32, msl=8192,
             topk=16, I=1, L=2, out=FAKE * 6, oh=32 * 16, orow=16)
    d.update(kw)
    return B.lib().mm3_index_topk_blocks(d["scores"], d["sh"], d["sr"], d["sw"], d["heads"], d["rb"],
                                         d["T"], d["msl"], d["topk"], d["I"], d["L"], d["out"],
                                         d["oh"], d["orow"], None)


BAD_TOPK_BLOCKS = [
    ("null_blocks", dict(rb=None), "row_blocks"),
    ("blocks_misaligned", dict(rb=FAKE * 4 + 2), "aligned"),
    ("negative_rows", dict(T=-1), "total_q"),
    ("rows_past_grid_bound", dict(T=(1 << 31) - 1023), "2^31 - 1024"),
    ("forced_exceed", dict(topk=4, I=3, L=2, orow=4, oh=128), "exceeds"),
    ("score_width", dict(sw=10, sr=10, sh=320), "width"),
    ("head_stride", dict(sh=31 * 64), "head stride"),
    ("out_row_stride", dict(orow=8), "row stride"),
]


@pytest.mark.parametrize("label,kw,msg", BAD_TOPK_BLOCKS, ids=[b[0] for b in BAD_TOPK_BLOCKS])
def test_topk_blocks_rules(label, kw, msg):
    assert _topk_blocks(**kw) == B.MM3_EINVAL
    assert msg in _err(), _err()


def _selector(s_ptr=FAKE, sh=None, sr=128, sw=128, heads=4, T=32768, msl=16384, topk=16, rowb=0,
              sparse=0):
    sh = T * sr if sh is None else sh
    r = B.lib().mm3_index_topk_selector(s_ptr, sh, sr, sw, heads, T, msl, topk, rowb, sparse)
    return None if r is None else r.decode()


@pytest.mark.parametrize("kw,want", [
    # chunked-prefill shape: 131072 (row, head) pairs of 128 blocks -> two lanes per row
    (dict(), "topk_lanes_kernel<4, false, 2>"),
    (dict(rowb=1), "topk_lanes_kernel<4, true, 2>"),
    # topk above the lanes' kept list -> several rows per wave, two keys per lane
    (dict(topk=20), "topk_kernel<2, false, 4, false>"),
    (dict(topk=20, rowb=1), "topk_kernel<2, false, 4, true>"),
    # rows past 512 blocks -> the wave-per-row search, 16 keys per lane
    (dict(msl=70000, sw=560, sr=560), "topk_kernel<16, false, 4, false>"),
    # a decode batch: one row per wave
    (dict(heads=4, T=256, msl=32768, sw=256, sr=256), "topk_kernel<4, false, 1, false>"),
    # the fused sparse table: one head, one row per wave, the sparse form
    (dict(heads=1, T=1024, msl=131072, sw=1024, sr=1024, sparse=1), "topk_kernel<16, true, 1, false>"),
    # rows past 1024 blocks re-read the score row
    (dict(heads=1, T=8, msl=200000, sw=1568, sr=1568), "topk_kernel<0, false, 1, false>"),
    # unaligned scores cannot take the lanes' 16-byte loads
    (dict(s_ptr=FAKE + 4), "topk_kernel<2, false, 4, false>"),
    # no row sees a block: no selector reads scores
    (dict(msl=0, sw=0, sr=0), "no_blocks_kernel"),
])
def test_selector_query_names_the_launched_kernel(kw, want):
    assert _selector(**kw) == want


def _launches(p, scores=None, sh=0, sr=0, sparse=None):
    return B.lib().mm3_index_decode_launches(ctypes.byref(p), scores, sh, sr,
                                             None if sparse is None else ctypes.byref(sparse))


@pytest.mark.parametrize("kw,want", [
    # 8 requests of 4 heads x 4 rows that see at most 16 blocks: one launch
    (dict(max_seq_len=2048), 1),
    (dict(max_seq_len=2049), 2),              # 17 blocks
    (dict(max_seq_len=2048, num_reqs=256), 1),
    (dict(max_seq_len=2048, num_reqs=257), 2),
    (dict(max_seq_len=2048, heads=8), 2),     # 32 rows per request: the prefill scorer
    (dict(max_seq_len=2048, heads=16, query_len=1, q_tok_stride=16 * 128), 1),
    (dict(max_seq_len=0), 2),                 # no block: the selector alone writes the -1 rows
])
def test_decode_launches_query(kw, want):
    assert _launches(_problem(**kw)) == want


def test_decode_launches_query_scores_out_and_sparse():
    p = _problem(max_seq_len=2048)
    T = p.rows.total_q
    assert _launches(p, FAKE * 5, T * 16, 16) == 1
    # a score tensor past 2 GiB is not addressable through one buffer descriptor
    assert _launches(p, FAKE * 5, 1 << 29, 16) == 2
    assert _launches(p, sparse=B.SparseOut()) == 2
    assert _launches(_problem(heads=0)) == B.MM3_EINVAL
    assert "heads" in _err()


def test_selector_query_rejects_invalid():
    assert _selector(topk=0) is None
    assert "topk" in B.lib().mm3_last_error().decode()
    assert _selector(sw=100) is None  # narrower than cdiv(16384, 128)
    assert _selector(heads=4, sparse=1) is None
    assert _selector(msl=65535 * 128) is None


def test_static_decode_validates_before_any_hip_call():
    """The no-allocation decode checks its arguments, and that the batch's
    scores fit the library's 64 MiB workspace, before touching the GPU."""
    lib = B.lib()
    out = ctypes.c_void_p(FAKE * 5)
    # 4 heads x 32800 rows x 128 blocks of scores: past 64 MiB
    p = _problem(heads=4, num_reqs=4, query_len=8200, max_seq_len=16384, bt_width=128,
                 bt_row_stride=128)
    rc = lib.mm3_index_decode_static(ctypes.byref(p), 16, 1, 2, out, 32800 * 16, 16, None, 0, 0, 0,
                                     None, None)
    assert rc == B.MM3_EWORKSPACE
    msg = lib.mm3_last_error().decode()
    assert "67174400" in msg and str(B.STATIC_SCRATCH_BYTES) in msg
    p = _problem(heads=4)
    rc = lib.mm3_index_decode_static(ctypes.byref(p), 0, 0, 0, out, 32 * 16, 16, None, 0, 0, 0,
                                     None, None)
    assert rc == B.MM3_EINVAL and "topk" in lib.mm3_last_error().decode()


def test_fused_prefill_workspace_sizes():
    """The fused prefill selection asks for two int32 words per (request,
    512-row tile) after the scores; mm3_index_decode asks for the scores
    only.  Decode batches, topk above 16 and rows past 512 blocks cannot take
    the fused call (MM3_EUNSUPPORTED, size 0)."""
    lib = B.lib()
    dec_ws = lambda p, k=16, so=0: lib.mm3_index_decode_workspace_bytes(ctypes.byref(p), k, so)
    sel_ws = lambda p, k=16, so=0: lib.mm3_index_prefill_select_workspace_bytes(ctypes.byref(p), k, so)
    r256 = lambda n: -(-n // 256) * 256
    p = _problem(heads=4, num_reqs=4, query_len=8192, max_seq_len=16384, bt_width=128,
                 bt_row_stride=128)
    units = 4 * 64  # 4 requests x (4 * 8192 / 512) row tiles
    assert dec_ws(p) == r256(4 * 32768 * 128 * 4)
    assert sel_ws(p) == r256(4 * 32768 * 128 * 4) + r256(2 * units * 4)
    assert sel_ws(p, so=1) == r256(2 * units * 4)
    assert sel_ws(p, k=17) == 0 and "topk <= 16" in lib.mm3_last_error().decode()
    wide = _problem(heads=4, num_reqs=4, query_len=8192, max_seq_len=65537, bt_width=513,
                    bt_row_stride=513)
    assert sel_ws(wide, so=1) == 0
    dec = _problem(heads=4, num_reqs=8, query_len=4, max_seq_len=8192)
    assert sel_ws(dec, so=1) == 0
    out = ctypes.c_void_p(FAKE * 5)
    rc = lib.mm3_index_prefill_select(ctypes.byref(dec), 16, 1, 2, out, 32 * 16, 16, None, 0, 0, 0,
                                      ctypes.c_void_p(FAKE * 6), 1 << 20, None)
    assert rc == B.MM3_EUNSUPPORTED
    rc = lib.mm3_index_prefill_select(ctypes.byref(p), 16, 1, 2, out, 32768 * 16, 16, None, 0, 0, 0,
                                      ctypes.c_void_p(FAKE * 6), 1 << 20, None)
    assert rc == B.MM3_EWORKSPACE


def test_fused_prefill_empty_batch_succeeds():
    """No rows: nothing to score or select, no workspace needed, MM3_OK (as
    every entry point does for an empty batch)."""
    lib = B.lib()
    p = _problem(heads=4, num_reqs=0, query_len=700, total_q=0, max_seq_len=8192)
    assert lib.mm3_index_prefill_select_workspace_bytes(ctypes.byref(p), 16, 0) == 0
    assert lib.mm3_last_error().decode() == ""
    rc = lib.mm3_index_prefill_select(ctypes.byref(p), 16, 1, 2, ctypes.c_void_p(FAKE * 5), 0, 16,
                                      None, 0, 0, 0, None, 0, None)
    assert rc == B.MM3_OK
