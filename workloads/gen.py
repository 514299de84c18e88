"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no arithmetic of the method (no dot products, maxima,
dequantisation or selection).  It only draws inputs: index queries, a paged
index-K pool (bf16, or NVFP4 codes), a block table of randomly permuted pages
and sequence lengths.  Both the HIP path and the CPU oracle consume what it
returns; neither imports the other.

Shapes follow the pages: queries [tokens, heads, 128] bf16, index-K pages
[pages, 128, 128] bf16 with one page per 128-token block, int32 block table
and lengths, query_len rows per request (page "ops.index_topk", module
docstring; page "indexer_context_parallel", check_context_score_inputs), or
ragged batches with cu_seqlens_q row offsets and optional prefix_lens (page
"ops.index_topk", minimax_m3_index_score signature).
NVFP4 keys are e2m1 nibbles with one e4m3 scale per 16 elements (page
"indexer_nvfp4", module docstring).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BLOCK = 128
DIM = 128
KFMT_BF16 = 0
KFMT_NVFP4 = 1

# Poison written into K slots no correct kernel may read: the tail tokens of
# a request's last, partial page and every page the block table maps to no
# visible block.  A read of it shows up as a huge block score.
POISON_BF16 = 1.0e4
POISON_NIB = 0x7  # e2m1 +6
POISON_SCALE = 0x7E  # e4m3 448


@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor  # [T, H, 128] bf16
    kfmt: int
    kdata: torch.Tensor  # bf16 [P,128,128] or uint8 [P,128,64]
    kscales: Optional[torch.Tensor]  # uint8 [P,128,8] or None
    block_table: torch.Tensor  # int32 [R, W]
    seq_lens: torch.Tensor  # int32 [R]
    query_len: int  # rows per request; ragged: the bound on every request's rows
    max_seq_len: int
    sm_scale: float
    topk: int
    init_blocks: int
    local_blocks: int
    cu_seqlens_q: Optional[torch.Tensor] = None  # int32 [R+1] (ragged batches)
    prefix_lens: Optional[torch.Tensor] = None  # int32 [R] (position of a request's first row)

    @property
    def ragged(self) -> bool:
        return self.cu_seqlens_q is not None

    def row_ranges(self):
        """[(first row, rows)] per request (host ints)."""
        if self.cu_seqlens_q is None:
            return [(r * self.query_len, self.query_len) for r in range(self.num_reqs)]
        cu = self.cu_seqlens_q.detach().cpu().tolist()
        return [(cu[r], cu[r + 1] - cu[r]) for r in range(self.num_reqs)]

    @property
    def num_reqs(self) -> int:
        return int(self.seq_lens.numel())

    @property
    def heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def nb_max(self) -> int:
        return cdiv(self.max_seq_len, BLOCK)

    @property
    def score_width(self) -> int:
        return round_up(self.nb_max, 16)

    def key_bytes_per_token(self) -> int:
        return 2 * DIM if self.kfmt == KFMT_BF16 else DIM // 2 + DIM // 16

    def to(self, device) -> "Workload":
        f = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(
            self, q=f(self.q), kdata=f(self.kdata), kscales=f(self.kscales),
            block_table=f(self.block_table), seq_lens=f(self.seq_lens),
            cu_seqlens_q=f(self.cu_seqlens_q), prefix_lens=f(self.prefix_lens))


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def round_up(a: int, b: int) -> int:
    return cdiv(a, b) * b


# The five workloads: (name, R, len range, Q, H, max_seq_len, topk, I, L,
# key format, extras).  Each workload is seeded with its number.
WORKLOADS = {
    1: dict(name="tiny_decode", R=1, lens=(1000, 1000), Q=4, H=1,
            max_seq_len=2048, topk=4, I=1, L=1, kfmt=KFMT_BF16, pool=16),
    2: dict(name="decode_batch", R=64, lens=(4096, 32768), Q=4, H=4,
            max_seq_len=32768, topk=16, I=1, L=2, kfmt=KFMT_BF16,
            dup_frac=0.01),
    3: dict(name="long_decode", R=256, lens=(32768, 131072), Q=4, H=1,
            max_seq_len=131072, topk=16, I=1, L=2, kfmt=KFMT_BF16,
            block_sigma=0.5),
    4: dict(name="chunked_prefill", R=4, lens=(16384, 16384), Q=8192, H=4,
            max_seq_len=16384, topk=16, I=1, L=2, kfmt=KFMT_BF16),
    5: dict(name="nvfp4_decode", R=128, lens=(16384, 65536), Q=4, H=1,
            max_seq_len=65536, topk=16, I=1, L=2, kfmt=KFMT_NVFP4),
    # beyond the five: the chunked-prefill shape with NVFP4 keys
    6: dict(name="chunked_prefill_nvfp4", R=4, lens=(16384, 16384), Q=8192, H=4,
            max_seq_len=16384, topk=16, I=1, L=2, kfmt=KFMT_NVFP4),
    # a ragged serving batch: 64 decode requests of 1..4 speculative rows and
    # two 4096-token prefill chunks, in one call (cu_seqlens_q, prefix_lens)
    7: dict(name="mixed_serving", R=66, lens=(4096, 32768), Q=4096, H=4,
            max_seq_len=32768, topk=16, I=1, L=2, kfmt=KFMT_BF16,
            qlens=[(1, 4)] * 64 + [4096, 4096], prefix="tail"),
}


def config(cid: int, device="cpu", seed: Optional[int] = None, **override) -> Workload:
    c = dict(WORKLOADS[cid])
    c.update(override)
    return make(seed=cid if seed is None else seed, device=device, **c)


def _quantize_nvfp4(x: torch.Tensor):
    """Generator-side NVFP4 encoder: per 16-element group, scale code
    s = e4m3(amax/6) by torch's round-to-nearest-even fp8 cast, then each
    element's e2m1 code by round-to-nearest-even of x/s with saturation at 6.
    Only the resulting codes are inputs; the path decodes them."""
    shp = x.shape
    g = x.reshape(*shp[:-1], DIM // 16, 16).float()
    amax = g.abs().amax(-1)
    s8 = (amax / 6.0).to(torch.float8_e4m3fn)
    sv = s8.float().unsqueeze(-1)
    v = torch.where(sv > 0, g / torch.where(sv > 0, sv, torch.ones_like(sv)),
                    torch.zeros_like(g))
    mag = v.abs()
    code = torch.zeros_like(mag, dtype=torch.int32)
    # thresholds between neighbouring e2m1 magnitudes; ties go to the even code
    code = torch.where(mag > 0.25, 1, code)
    code = torch.where(mag >= 0.75, 2, code)
    code = torch.where(mag > 1.25, 3, code)
    code = torch.where(mag >= 1.75, 4, code)
    code = torch.where(mag > 2.5, 5, code)
    code = torch.where(mag >= 3.5, 6, code)
    code = torch.where(mag > 5.0, 7, code)
    code = code | (torch.signbit(v).to(torch.int32) << 3)
    code = code.reshape(*shp[:-1], DIM)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).to(torch.uint8)
    scales = s8.view(torch.uint8)
    return packed, scales


def make(name, R, lens, Q, H, max_seq_len, topk, I, L, kfmt, seed, device,
         pool=None, dup_frac=0.0, block_sigma=0.0, fixed_lens=None,
         sm_scale=None, poison=True, chunk_pages=4096, qlens=None,
         prefix=None, max_gap=300) -> Workload:
    """Draw one workload.  Lengths ~ U[lens[0], lens[1]] (integers); pages
    are a seeded random permutation of a pool of sum(cdiv(len,128)) pages
    (plus one page that only the unused block-table entries point at);
    q, k ~ N(0,1) rounded to bf16; NVFP4 keys are N(0,1) values encoded by
    _quantize_nvfp4.

    Ragged batches: qlens gives each request's row count, as one (lo, hi)
    range drawn uniformly per request, or as a list of counts and ranges, one
    per request; Q is then the bound on them
    (cu_seqlens_q holds the row offsets).  prefix: None (no prefix_lens: a
    request's rows are its last tokens), "tail" (prefix_lens = seq_len -
    rows, passed explicitly) or "gap" (prefix_lens = seq_len - rows - gap,
    gap ~ U[0, max_gap]: the keys after the last row's position exist but no
    row sees them; they are poisoned).  With a prefix, rows are capped at
    seq_len."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    W = cdiv(max_seq_len, BLOCK)
    if fixed_lens is not None:
        seq = torch.as_tensor(fixed_lens, dtype=torch.int64).to(dev)
        assert seq.numel() == R
    else:
        seq = torch.randint(lens[0], lens[1] + 1, (R,), generator=g, device=dev)
    seq_host = seq.cpu().tolist()
    assert max(seq_host + [0]) <= max_seq_len
    cu = pre = None
    if qlens is not None:
        spec = [qlens] * R if isinstance(qlens, tuple) else list(qlens)
        assert len(spec) == R
        lo = torch.tensor([x[0] if isinstance(x, tuple) else int(x) for x in spec])
        hi = torch.tensor([x[1] if isinstance(x, tuple) else int(x) for x in spec])
        u = torch.rand((R,), generator=g, device=dev).cpu().double()
        nq = (lo + (u * (hi - lo + 1).double()).floor().long().clamp(max=(hi - lo))).tolist()
        if prefix is not None:
            nq = [min(n, s) for n, s in zip(nq, seq_host)]
        assert max(nq + [0]) <= Q
        cu_host = [0]
        for n in nq:
            cu_host.append(cu_host[-1] + n)
        cu = torch.tensor(cu_host, dtype=torch.int32, device=dev)
        if prefix is not None:
            assert prefix in ("tail", "gap")
            gaps = [0] * R
            if prefix == "gap":
                gaps = torch.randint(0, max_gap + 1, (R,), generator=g, device=dev).cpu().tolist()
            pre_host = [max(0, s - n - gp) for s, n, gp in zip(seq_host, nq, gaps)]
            pre = torch.tensor(pre_host, dtype=torch.int32, device=dev)
        T = cu_host[-1]
    else:
        assert prefix is None and Q >= 1
        T = R * Q
    nblk = [cdiv(s, BLOCK) for s in seq_host]
    used = sum(nblk)
    npages = max(used + 1, pool or 0)
    perm = torch.randperm(npages, generator=g, device=dev).to(torch.int32)
    if R == 1 and npages == W:
        bt = perm.view(1, W).clone()
    else:
        bt = torch.empty((R, W), dtype=torch.int32, device=dev)
        bt.fill_(0)
        bt[:] = perm[used]
        off = 0
        for r, nb in enumerate(nblk):
            bt[r, :nb] = perm[off:off + nb]
            off += nb
    q = torch.randn((T, H, DIM), generator=g, device=dev).to(torch.bfloat16)

    # K pool, drawn in chunks of pages to bound the fp32 temporary
    if kfmt == KFMT_BF16:
        kdata = torch.empty((npages, BLOCK, DIM), dtype=torch.bfloat16, device=dev)
        kscales = None
    else:
        kdata = torch.empty((npages, BLOCK, DIM // 2), dtype=torch.uint8, device=dev)
        kscales = torch.empty((npages, BLOCK, DIM // 16), dtype=torch.uint8, device=dev)
    for p0 in range(0, npages, chunk_pages):
        p1 = min(npages, p0 + chunk_pages)
        x = torch.randn((p1 - p0, BLOCK, DIM), generator=g, device=dev)
        if block_sigma:
            x += block_sigma * torch.randn((p1 - p0, 1, 1), generator=g, device=dev)
        if kfmt == KFMT_BF16:
            kdata[p0:p1] = x.to(torch.bfloat16)
        else:
            kdata[p0:p1], kscales[p0:p1] = _quantize_nvfp4(x)
        del x

    if dup_frac:
        _duplicate_keys(kdata, kscales, bt, seq_host, dup_frac, g, dev)

    if poison:
        bt_host = bt.cpu()
        mapped = torch.zeros(npages, dtype=torch.bool)
        for r, nb in enumerate(nblk):
            mapped[bt_host[r, :nb].long()] = True
        unused = (~mapped).nonzero().flatten().to(dev)
        if unused.numel():
            _fill_poison(kdata, kscales, unused, slice(None))
        for r, s in enumerate(seq_host):
            tail = s % BLOCK
            if s > 0 and tail:
                page = int(bt_host[r, nblk[r] - 1])
                _fill_poison(kdata, kscales, torch.tensor([page], device=dev),
                             slice(tail, BLOCK))
        if pre is not None:
            # keys after the last row's position: present, seen by no row
            for r, (p0, s) in enumerate(zip(pre.cpu().tolist(), seq_host)):
                end = p0 + cu_host[r + 1] - cu_host[r]
                for p in range(end, s):
                    page = int(bt_host[r, p // BLOCK])
                    _fill_poison(kdata, kscales, torch.tensor([page], device=dev),
                                 slice(p % BLOCK, p % BLOCK + 1))

    return Workload(
        name=name, q=q, kfmt=kfmt, kdata=kdata, kscales=kscales,
        block_table=bt, seq_lens=seq.to(torch.int32), query_len=Q,
        max_seq_len=max_seq_len,
        sm_scale=float(1.0 / math.sqrt(DIM)) if sm_scale is None else float(sm_scale),
        topk=topk, init_blocks=I, local_blocks=L, cu_seqlens_q=cu, prefix_lens=pre)


def _fill_poison(kdata, kscales, pages, toks):
    if kscales is None:
        kdata[pages, toks] = POISON_BF16
    else:
        kdata[pages, toks] = POISON_NIB | (POISON_NIB << 4)
        kscales[pages, toks] = POISON_SCALE


def _duplicate_keys(kdata, kscales, bt, seq_host, frac, g, dev):
    """Overwrite a fraction of each request's visible key slots with copies
    of keys from another block of the same request (forces score ties)."""
    btl = bt.long()
    for r, s in enumerate(seq_host):
        n = max(1, int(round(frac * s)))
        dst = torch.randint(0, s, (n,), generator=g, device=dev)
        src = torch.randint(0, s, (n,), generator=g, device=dev)
        same = (src // BLOCK) == (dst // BLOCK)
        src = torch.where(same, (src + BLOCK) % s, src)
        same = (src // BLOCK) == (dst // BLOCK)
        src = torch.where(same, (src + 2 * BLOCK) % s, src)
        dp, dt = btl[r, dst // BLOCK], dst % BLOCK
        sp, st = btl[r, src // BLOCK], src % BLOCK
        kdata[dp, dt] = kdata[sp, st].clone()
        if kscales is not None:
            kscales[dp, dt] = kscales[sp, st].clone()


# --------------------------------------------------------------- host views

def host_arrays(w: Workload):
    """The workload as host numpy arrays in the oracle's form (bf16 as
    uint16 bit patterns)."""
    q = w.q.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    if w.kfmt == KFMT_BF16:
        kd = w.kdata.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        ks = None
    else:
        kd = w.kdata.detach().cpu().contiguous().numpy()
        ks = w.kscales.detach().cpu().contiguous().numpy()
    f = lambda t: None if t is None else t.detach().cpu().numpy()
    return dict(q_bits=q, kfmt=w.kfmt, kdata=kd, kscales=ks,
                block_table=w.block_table.detach().cpu().numpy(),
                seq_lens=w.seq_lens.detach().cpu().numpy(),
                query_len=w.query_len, sm_scale=w.sm_scale,
                cu_seqlens_q=f(w.cu_seqlens_q), prefix_lens=f(w.prefix_lens))


def host_subset(w: Workload, reqs, max_pages_per_req=None):
    """Host arrays for a subset of requests: only the pages their visible
    blocks map to are copied (device -> host), into a compact pool with a
    remapped block table.  Returns (arrays, row_index) where row_index maps
    the subset's rows back to rows of the full workload."""
    reqs = [int(r) for r in reqs]
    Q = w.query_len
    ranges = w.row_ranges()
    seq = w.seq_lens.detach().cpu()
    bt = w.block_table.detach().cpu()
    pages, tables = [], []
    for r in reqs:
        nb = cdiv(int(seq[r]), BLOCK)
        tables.append(bt[r, :nb].long())
    allp = torch.cat(tables) if tables else torch.zeros(0, dtype=torch.long)
    uniq, inv = torch.unique(allp, return_inverse=True)
    W = max([t.numel() for t in tables] + [1])
    nbt = torch.zeros((len(reqs), W), dtype=torch.int32)
    off = 0
    for i, t in enumerate(tables):
        nbt[i, :t.numel()] = inv[off:off + t.numel()].to(torch.int32)
        off += t.numel()
    dev_idx = uniq.to(w.kdata.device)
    rows = (torch.cat([torch.arange(ranges[r][0], ranges[r][0] + ranges[r][1]) for r in reqs])
            if reqs else torch.zeros(0, dtype=torch.long))
    q = w.q.index_select(0, rows.to(w.q.device)).cpu().contiguous()
    q = q.view(torch.int16).numpy().view(np.uint16)
    if w.kfmt == KFMT_BF16:
        kd = w.kdata.index_select(0, dev_idx).cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        ks = None
    else:
        kd = w.kdata.index_select(0, dev_idx).cpu().contiguous().numpy()
        ks = w.kscales.index_select(0, dev_idx).cpu().contiguous().numpy()
    cu = pre = None
    if w.ragged:
        cu = np.cumsum([0] + [ranges[r][1] for r in reqs]).astype(np.int32)
        if w.prefix_lens is not None:
            pre = w.prefix_lens.detach().cpu().numpy()[reqs].astype(np.int32)
    arrays = dict(q_bits=q, kfmt=w.kfmt, kdata=kd, kscales=ks,
                  block_table=nbt.numpy(), seq_lens=seq[reqs].numpy().astype(np.int32),
                  query_len=Q, sm_scale=w.sm_scale, cu_seqlens_q=cu, prefix_lens=pre)
    return arrays, rows.numpy()
