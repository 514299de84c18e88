"""The work model behind bench.py's roofline figures, pinned by hand counts.

The "achieved" rate in the benchmark line is algorithmic bytes (decode scorer)
or flops (prefill scorer) divided by measured time.  These cases count the
work by hand from the definitions: the decode scorer's unit is bytes (every
visible key once, the query rows, the block-table entries, the scores
written), and the prefill scorer's unit is 2 * 128 flops per (row, head,
visible key).
"""
import pytest

import bench
from workloads import make


def _seq(w):
    return w.seq_lens.cpu().numpy()


def test_tiny_decode_bytes_by_hand():
    # one request of 1000 tokens, 4 decode rows at positions 996..999, 1 head
    w = make("hand", R=1, lens=(1000, 1000), Q=4, H=1, max_seq_len=2048, topk=4, I=1, L=1,
             kfmt=0, seed=3, device="cpu", fixed_lens=[1000])
    a = bench.algorithmic(w, _seq(w))
    keys = 1000 * 256           # 1000 visible keys of 128 bf16
    q = 4 * 1 * 256             # 4 rows x 1 head x 128 bf16
    table = 8 * 4               # cdiv(1000, 128) block-table entries
    scores = 4 * 8 * 4          # each row sees 996 // 128 + 1 = 8 blocks
    assert a["k_bytes"] == keys
    assert a["scorer_bytes"] == keys + q + table + scores
    assert a["flops"] == 0
    assert a["tokens"] == 1000
    assert a["rows"] == 4
    assert a["selector_bytes"] == scores + 4 * 4 * 4   # scores read + [1, 4, 4] ids


def test_nvfp4_keys_count_72_bytes_per_token():
    w = make("hand", R=1, lens=(640, 640), Q=2, H=2, max_seq_len=1024, topk=4, I=1, L=1,
             kfmt=1, seed=4, device="cpu", fixed_lens=[640])
    a = bench.algorithmic(w, _seq(w))
    assert a["k_bytes"] == 640 * 72
    nv = 2 * (638 // 128 + 1)   # rows at 638, 639: 5 blocks each
    assert a["scorer_bytes"] == 640 * 72 + 2 * 2 * 256 + 5 * 4 + 2 * nv * 4


def test_prefill_flops_by_hand():
    # 8 rows x 4 heads = 32 > 16 rows: the prefill scorer's request
    w = make("hand", R=1, lens=(300, 300), Q=8, H=4, max_seq_len=512, topk=4, I=1, L=1,
             kfmt=0, seed=5, device="cpu", fixed_lens=[300])
    a = bench.algorithmic(w, _seq(w))
    visible = sum(p + 1 for p in range(292, 300))   # rows at positions 292..299
    assert a["flops"] == 2 * 128 * 4 * visible
    assert a["scorer_bytes"] == 0
    assert a["pairs"] == 4 * visible


def test_mixed_batch_splits_by_row_count():
    # request 0: 2 rows x 4 heads = 8 <= 16 (decode); request 1: 8 rows x 4 = 32 (prefill)
    w = make("hand", R=2, lens=(256, 256), Q=8, H=4, max_seq_len=512, topk=4, I=1, L=1,
             kfmt=0, seed=6, device="cpu", fixed_lens=[256, 300], qlens=[2, 8], prefix="tail")
    a = bench.algorithmic(w, _seq(w))
    dec_keys = 256 * 256
    dec = dec_keys + 2 * 4 * 256 + 2 * 4 + 4 * 2 * 2 * 4   # rows at 254, 255: 2 blocks each
    assert a["scorer_bytes"] == dec
    assert a["k_bytes"] == dec_keys
    assert a["flops"] == 2 * 128 * 4 * sum(p + 1 for p in range(292, 300))
    assert a["tokens"] == 256 + 300


def test_bench_refuses_several_gpus(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_selector_kernel_follows_the_launch_rule():
    # the benchmark names the selector kernel the library itself reports for
    # the batch (mm3_index_topk_selector): lanes selecting rows by themselves
    # for topk <= 16, from 65536, 24576, 16384 or 8192 (head, row) pairs for
    # rows of up to 64, 128, 256 or 512 blocks, else one wave per row
    from sparse_attention_block_paged_amd import _binding as B

    def name(heads, rows, topk, max_seq_len):
        w = -(-(-(-max_seq_len // 128)) // 16) * 16
        r = B.lib().mm3_index_topk_selector(1 << 20, rows * w, w, w, heads, rows, max_seq_len, topk,
                                            0, 0)
        return r.decode().split("<")[0]

    lanes = [(4, 32768, 16, 16384),     # chunked prefill
             (4, 8352, 16, 32768),      # mixed serving
             (4, 8192, 16, 65536),      # 512 blocks
             (4, 6144, 16, 16384),      # 24576 pairs, 128 blocks
             (4, 16384, 16, 8192)]      # 65536 pairs, 64 blocks
    ballot = [(4, 256, 16, 32768),      # decode batch
              (1, 512, 16, 65536),      # NVFP4 decode
              (1, 1024, 16, 131072),    # long decode
              (4, 8192, 16, 8192),      # 32768 pairs, 64 blocks
              (4, 4096, 16, 16384),     # 16384 pairs, 128 blocks
              (4, 32768, 16, 65537),    # 513 blocks
              (4, 32768, 17, 16384)]    # topk 17
    for w in lanes:
        assert name(*w) == "topk_lanes_kernel", w
    for w in ballot:
        assert name(*w) == "topk_kernel", w
