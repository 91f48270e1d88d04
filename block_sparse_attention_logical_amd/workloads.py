"""Seeded synthetic workloads shaped like the LServe evaluations.

This module only makes inputs: random tensors, page tables, head classes,
outlier channels, needle keys and the int4 storage of the KV pool.  It holds
none of the attention method's arithmetic (no statistics, scores, selection or
softmax), and it is the only code shared by the GPU tests and the oracle.

Recipe (fixed order of random draws from one torch.Generator seeded with the
config id, on the device the pool is built on):
  1. head classes: exactly H_kv/2 streaming KV heads, a seeded subset
     (config 1 is fixed: KV head 0 retrieval, KV head 1 streaming);
  2. outlier channels: 4 per KV head, shared by the batch (keys only, x8);
  3. context lengths (config 4: uniform in [128K, 256K]);
  4. the page table: identity, or a seeded permutation of all pool pages;
  5. queries of the decode window, N(0, 1);
  6. needle positions: 8 per sequence, uniform in [0, ctx); the needle key is
     3 * the unit vector of the sum of the group's step-0 queries;
  7. keys, page chunk by page chunk: N(0, 1), outlier channels x8, needles
     written over their slots, then int4 storage;
  8. values, page chunk by page chunk: N(0, 1), then int4 storage.
Prefill (configs 3 and 7): head classes, then per-head scales U[0.5, 2] for
q, k and v, then q, k, v ~ N(0, 1) * scale.
Configs 6 (decode) and 7 (prefill) are multi-head attention (32 query heads,
32 KV heads, group size 1) with the other settings of configs 2 and 3.

int4 storage (KV4): per (pool page, KV head, tensor) scale s = fp16 of
(max - min) / 15 (at least 2^-10) and zero point z = round(16 * (-min / s)) / 16
clamped to [0, 15], so (c - z) * s is exact in fp32; codes
c = clamp(round(x / s + z), 0, 15); keys packed two channels per byte (even
channel in the low nibble), values two tokens per byte.

Every pool is written in the library's page layout: keys as BT x 32 tiles
[P][H_kv][N_P/BT][D/32][BT][32], values as rows [P][H_kv][N_P/BT][D][BT],
BT = min(N_P, 32) (int4: the same with code pairs packed into bytes).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

F32, BF16, INT4 = 0, 1, 2


@dataclass
class DecodeWorkload:
    cfg: int
    dtype: int                    # F32 | BF16 | INT4 (KV storage); q is f32 for F32, else bf16
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    logical_page: int
    page_size: int
    token_budget: int
    reuse_interval: int
    sink_tokens: int
    local_tokens: int
    sink_blocks: int
    local_blocks: int
    head_kind: List[int]
    ctx: List[int]                # cached tokens before the decode window
    window: int                   # decode steps
    max_pages: int
    num_pages: int
    page_table: torch.Tensor      # int32 [B][max_pages]
    k: torch.Tensor
    v: torch.Tensor
    q: torch.Tensor               # [window][B][H_q][D]
    k_sz: Optional[torch.Tensor] = None   # int4: [P][H_kv][2] fp16
    v_sz: Optional[torch.Tensor] = None
    outliers: Optional[torch.Tensor] = None
    needles: Optional[torch.Tensor] = None   # [B][8] token positions

    def seq_lens(self, step: int) -> torch.Tensor:
        """Tokens in cache at decode step `step` (the step's token included)."""
        return torch.tensor([c + step + 1 for c in self.ctx], dtype=torch.int32, device=self.page_table.device)


@dataclass
class PrefillWorkload:
    cfg: int
    dtype: int
    seq_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    logical_page: int
    sink_blocks: int
    local_blocks: int
    head_kind: List[int]
    num_pages: int
    page_table: torch.Tensor      # int32 [ceil(T / N_P)]
    q: torch.Tensor               # [T][H_q][D]
    k: torch.Tensor
    v: torch.Tensor
    scales: dict = field(default_factory=dict)


# ---------------------------------------------------------------------------
# config table
# ---------------------------------------------------------------------------

DECODE_CONFIGS = {
    1: dict(dtype=F32, batch=1, num_q_heads=4, num_kv_heads=2, head_dim=64, logical_page=16, page_size=64,
            token_budget=256, reuse_interval=4, sink_tokens=16, local_tokens=128, sink_blocks=1, local_blocks=2,
            ctx=1024, window=16, permute=True, outliers=False, needles=0),
    2: dict(dtype=BF16, batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128, logical_page=16, page_size=64,
            token_budget=4096, reuse_interval=4, sink_tokens=64, local_tokens=1024, sink_blocks=1, local_blocks=16,
            ctx=65536, window=4, permute=False, outliers=True, needles=8),
    4: dict(dtype=BF16, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, logical_page=16, page_size=128,
            token_budget=4096, reuse_interval=4, sink_tokens=128, local_tokens=2048, sink_blocks=1, local_blocks=16,
            ctx=(131072, 262144), window=4, permute=True, outliers=True, needles=8),
    5: dict(dtype=INT4, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128, logical_page=16, page_size=64,
            token_budget=4096, reuse_interval=4, sink_tokens=64, local_tokens=1024, sink_blocks=1, local_blocks=16,
            ctx=262144, window=4, permute=False, outliers=True, needles=8),
    # multi-head attention (Llama-2-7B-shaped layer: 32 query heads, each its own KV head)
    6: dict(dtype=BF16, batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128, logical_page=16, page_size=64,
            token_budget=4096, reuse_interval=4, sink_tokens=64, local_tokens=1024, sink_blocks=1, local_blocks=16,
            ctx=65536, window=4, permute=False, outliers=True, needles=8),
}

PREFILL_CONFIGS = {
    1: dict(dtype=F32, seq_len=1024, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=64, logical_page=16,
            sink_blocks=1, local_blocks=2, permute=True, head_scales=False),
    3: dict(dtype=BF16, seq_len=131072, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
            logical_page=16, sink_blocks=1, local_blocks=16, permute=False, head_scales=True),
    # multi-head attention (Llama-2-7B-shaped layer)
    7: dict(dtype=BF16, seq_len=131072, num_q_heads=32, num_kv_heads=32, head_dim=128, page_size=64,
            logical_page=16, sink_blocks=1, local_blocks=16, permute=False, head_scales=True),
}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _head_kinds(n_kv: int, g: torch.Generator, fixed=None) -> List[int]:
    if fixed is not None:
        return list(fixed)
    perm = torch.randperm(n_kv, generator=g, device=g.device).tolist()
    kinds = [0] * n_kv
    for h in perm[: n_kv // 2]:
        kinds[h] = 1
    return kinds


def quantize_int4(x: torch.Tensor):
    """int4 codes of x [..., A, Bd], one (s, z) per leading index over its last
    two dims: returns (codes uint8 [..., A, Bd], [..., 2] fp16 {s, z})."""
    lead = x.shape[:-2]
    flat = x.reshape(*lead, -1).float()
    lo = flat.amin(dim=-1)
    hi = flat.amax(dim=-1)
    s = ((hi - lo) / 15.0).clamp_min(2.0 ** -10).to(torch.float16)
    s32 = s.float()
    z = torch.round(16.0 * (-lo / s32)) / 16.0
    z = z.clamp(0.0, 15.0).to(torch.float16)        # multiples of 1/16 in [0, 15] are exact in fp16
    z32 = z.float()
    c = torch.round(x.float() / s32[..., None, None] + z32[..., None, None]).clamp(0, 15).to(torch.uint8)
    sz = torch.stack([s, z], dim=-1)
    return c, sz


def pack_int4(c: torch.Tensor) -> torch.Tensor:
    """Pairs of 4-bit codes along the last dim into bytes (even element low)."""
    return (c[..., 0::2] | (c[..., 1::2] << 4)).contiguous()


def tile_keys(x: torch.Tensor) -> torch.Tensor:
    """Keys [..., N_P, D] of pages -> the pool's key tiles [..., N_P/BT, D/32, BT, 32],
    BT = min(N_P, 32)."""
    *lead, NP, D = x.shape
    bt = min(NP, 32)
    return x.reshape(*lead, NP // bt, bt, D // 32, 32).transpose(-3, -2).contiguous()


def tile_values(x: torch.Tensor) -> torch.Tensor:
    """Values [..., D, N_P] (channel-major) of pages -> the pool's value rows [..., N_P/BT, D, BT]."""
    *lead, D, NP = x.shape
    bt = min(NP, 32)
    return x.reshape(*lead, D, NP // bt, bt).transpose(-3, -2).contiguous()


def make_decode(cfg: int, device="cpu", *, batch: Optional[int] = None, ctx=None, window: Optional[int] = None,
                seed: Optional[int] = None, replicas: int = 1, chunk_pages: int = 2048,
                page_size: Optional[int] = None, logical_page: Optional[int] = None,
                head_dim: Optional[int] = None, num_q_heads: Optional[int] = None,
                num_kv_heads: Optional[int] = None) -> DecodeWorkload:
    """Build a decode workload.  Overrides shrink a config for tests or change
    its page geometry (physical page size N_P, logical page size N_L) or its
    head shape."""
    c = dict(DECODE_CONFIGS[cfg])
    for key, val in (("page_size", page_size), ("logical_page", logical_page), ("head_dim", head_dim),
                     ("num_q_heads", num_q_heads), ("num_kv_heads", num_kv_heads)):
        if val is not None:
            c[key] = val
    B = batch if batch is not None else c["batch"]
    W = window if window is not None else c["window"]
    ctx_spec = ctx if ctx is not None else c["ctx"]
    H_q, H_kv, D, NP = c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["page_size"]
    G = H_q // H_kv
    dt = c["dtype"]
    g = _gen(device, cfg if seed is None else seed)

    kinds = _head_kinds(H_kv, g, fixed=[0, 1] if cfg == 1 else None)
    outl = torch.stack([torch.randperm(D, generator=g, device=device)[:4] for _ in range(H_kv)]) \
        if c["outliers"] else None
    if isinstance(ctx_spec, tuple):
        lo, hi = ctx_spec
        ctx_list = torch.randint(lo, hi + 1, (B,), generator=g, device=device).tolist()
    elif isinstance(ctx_spec, list):
        ctx_list = list(ctx_spec)
    else:
        ctx_list = [int(ctx_spec)] * B
    pages = [-(-(cl + W) // NP) for cl in ctx_list]
    max_pages = max(pages)
    P = sum(pages)
    pool_ids = torch.randperm(P, generator=g, device=device) if c["permute"] else torch.arange(P, device=device)
    table = torch.zeros((B, max_pages), dtype=torch.int32, device=device)
    off = 0
    for b in range(B):
        table[b, : pages[b]] = pool_ids[off: off + pages[b]].to(torch.int32)
        off += pages[b]

    qdt = torch.float32 if dt == F32 else torch.bfloat16
    q = torch.randn((W, B, H_q, D), generator=g, device=device).to(qdt)

    # needles: positions and key vectors
    n_needles = c["needles"]
    needle_pos = None
    needle_vec = None
    if n_needles:
        needle_pos = torch.stack([torch.randint(0, max(1, ctx_list[b]), (n_needles,), generator=g, device=device)
                                  for b in range(B)])
        qs = q[0].float().reshape(B, H_kv, G, D).sum(dim=2)             # [B][H_kv][D]
        needle_vec = 3.0 * qs / qs.norm(dim=-1, keepdim=True)
        needle_pid = table.long().gather(1, needle_pos // NP)            # [B][n] pool pages
        needle_slot = needle_pos % NP
    kscale = torch.ones((H_kv, D), device=device)
    if outl is not None:
        kscale.scatter_(1, outl, 8.0)

    # keys, as tiles [P][H_kv][N_P/32][D/32][32][32] (int4: codes packed in pairs)
    bt = min(NP, 32)                  # tokens per layout block
    if dt == INT4:
        k = torch.empty((P, H_kv, NP // bt, D // 32, bt, 16), dtype=torch.uint8, device=device)
        k_sz = torch.empty((P, H_kv, 2), dtype=torch.float16, device=device)
    else:
        k = torch.empty((P, H_kv, NP // bt, D // 32, bt, 32), dtype=qdt, device=device)
        k_sz = None
    for p0 in range(0, P, chunk_pages):
        p1 = min(P, p0 + chunk_pages)
        x = torch.randn((p1 - p0, H_kv, NP, D), generator=g, device=device)
        x *= kscale[None, :, None, :]
        if n_needles:
            bi, ni = torch.nonzero((needle_pid >= p0) & (needle_pid < p1), as_tuple=True)
            if bi.numel():
                x[needle_pid[bi, ni] - p0, :, needle_slot[bi, ni], :] = needle_vec[bi]
        if dt == INT4:
            codes, sz = quantize_int4(x)
            k[p0:p1] = pack_int4(tile_keys(codes))
            k_sz[p0:p1] = sz
        else:
            k[p0:p1] = tile_keys(x.to(qdt))
    # values, drawn channel-major per page ([D][N_P]) and stored as rows
    # [P][H_kv][N_P/32][D][32] (int4: token codes packed in pairs)
    if dt == INT4:
        v = torch.empty((P, H_kv, NP // bt, D, bt // 2), dtype=torch.uint8, device=device)
        v_sz = torch.empty((P, H_kv, 2), dtype=torch.float16, device=device)
    else:
        v = torch.empty((P, H_kv, NP // bt, D, bt), dtype=qdt, device=device)
        v_sz = None
    for p0 in range(0, P, chunk_pages):
        p1 = min(P, p0 + chunk_pages)
        x = torch.randn((p1 - p0, H_kv, D, NP), generator=g, device=device)
        if dt == INT4:
            codes, sz = quantize_int4(x)
            v[p0:p1] = pack_int4(tile_values(codes))
            v_sz[p0:p1] = sz
        else:
            v[p0:p1] = tile_values(x.to(qdt))

    return DecodeWorkload(
        cfg=cfg, dtype=dt, batch=B, num_q_heads=H_q, num_kv_heads=H_kv, head_dim=D,
        logical_page=c["logical_page"], page_size=NP, token_budget=c["token_budget"],
        reuse_interval=c["reuse_interval"], sink_tokens=c["sink_tokens"], local_tokens=c["local_tokens"],
        sink_blocks=c["sink_blocks"], local_blocks=c["local_blocks"], head_kind=kinds, ctx=ctx_list,
        window=W, max_pages=max_pages, num_pages=P, page_table=table, k=k, v=v, q=q, k_sz=k_sz, v_sz=v_sz,
        outliers=outl, needles=needle_pos)


def make_prefill(cfg: int, device="cpu", *, seq_len: Optional[int] = None, seed: Optional[int] = None,
                 head_kind: Optional[List[int]] = None, num_kv_heads: Optional[int] = None,
                 head_dim: Optional[int] = None, page_size: Optional[int] = None,
                 num_q_heads: Optional[int] = None) -> PrefillWorkload:
    c = dict(PREFILL_CONFIGS[cfg])
    for key, val in (("num_kv_heads", num_kv_heads), ("head_dim", head_dim), ("page_size", page_size),
                     ("num_q_heads", num_q_heads)):
        if val is not None:
            c[key] = val
    T = seq_len if seq_len is not None else c["seq_len"]
    H_q, H_kv, D, NP = c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["page_size"]
    dt = c["dtype"]
    qdt = torch.float32 if dt == F32 else torch.bfloat16
    g = _gen(device, cfg if seed is None else seed)
    kinds = _head_kinds(H_kv, g, fixed=[0, 1] if cfg == 1 else None)
    if head_kind is not None:
        kinds = list(head_kind)
    P = -(-T // NP)
    table = (torch.randperm(P, generator=g, device=device) if c["permute"]
             else torch.arange(P, device=device)).to(torch.int32)
    if c["head_scales"]:
        sq = torch.rand(H_q, generator=g, device=device) * 1.5 + 0.5
        sk = torch.rand(H_kv, generator=g, device=device) * 1.5 + 0.5
        sv = torch.rand(H_kv, generator=g, device=device) * 1.5 + 0.5
    else:
        sq = torch.ones(H_q, device=device)
        sk = torch.ones(H_kv, device=device)
        sv = torch.ones(H_kv, device=device)
    q = (torch.randn((T, H_q, D), generator=g, device=device) * sq[None, :, None]).to(qdt)
    # pool pages are written through the page table: token p sits in page table[p // NP]
    k = torch.empty((P, H_kv, NP // 32, D // 32, 32, 32), dtype=qdt, device=device)
    v = torch.empty((P, H_kv, NP // 32, D, 32), dtype=qdt, device=device)
    kk = torch.randn((P, H_kv, NP, D), generator=g, device=device) * sk[None, :, None, None]
    k[table.long()] = tile_keys(kk.to(qdt))
    del kk
    vv = torch.randn((P, H_kv, D, NP), generator=g, device=device) * sv[None, :, None, None]
    v[table.long()] = tile_values(vv.to(qdt))
    del vv
    return PrefillWorkload(cfg=cfg, dtype=dt, seq_len=T, num_q_heads=H_q, num_kv_heads=H_kv, head_dim=D,
                           page_size=NP, logical_page=c["logical_page"], sink_blocks=c["sink_blocks"],
                           local_blocks=c["local_blocks"], head_kind=kinds, num_pages=P, page_table=table,
                           q=q, k=k, v=v, scales=dict(q=sq, k=sk, v=sv))


# ---------------------------------------------------------------------------
# static block masks (inputs of the CSR prefill)
# ---------------------------------------------------------------------------

def csr_from_tile_masks(masks) -> "tuple[torch.Tensor, torch.Tensor]":
    """Per-KV-head tile masks [H][n][n] (bool; row = query tile, column = key
    tile) -> row_ptr [H][n + 1] (offsets into one shared col_idx) and col_idx
    [nnz], int32 tensors on the CPU, key tiles ascending within a row."""
    m = torch.as_tensor(masks).bool().cpu()
    H, n, _ = m.shape
    offs = torch.zeros(H * n + 1, dtype=torch.int64)
    offs[1:] = torch.cumsum(m.sum(dim=2).reshape(-1), 0)
    row_ptr = torch.stack([offs[h * n: h * n + n + 1] for h in range(H)]).to(torch.int32)
    col_idx = m.nonzero()[:, 2].to(torch.int32).contiguous()     # (h, a, c) in lexicographic order
    return row_ptr.contiguous(), col_idx


def random_tile_masks(num_kv_heads: int, n_blocks: int, density: float, seed: int,
                      diagonal: bool = True) -> torch.Tensor:
    """Seeded random tile masks [H][n][n]: each tile below the diagonal kept
    with probability `density`, the diagonal tiles kept when `diagonal`."""
    g = torch.Generator().manual_seed(seed)
    m = torch.rand((num_kv_heads, n_blocks, n_blocks), generator=g) < density
    m = torch.tril(m, diagonal=-1)
    if diagonal:
        m |= torch.eye(n_blocks, dtype=torch.bool)[None]
    return m


# ---------------------------------------------------------------------------
# the streaming heads' constant-size cache and the token rows a decode step
# appends (input preparation: copies and gathers of the generated pool)
# ---------------------------------------------------------------------------

def retrieval_pool(w: DecodeWorkload):
    """The pool pages of the retrieval heads only ([P][H_r] pages, KV-head
    order), copied from a workload's every-head pool: (k, v, k_sz, v_sz)."""
    ret = torch.tensor([h for h in range(w.num_kv_heads) if w.head_kind[h] == 0], device=w.k.device)
    pick = lambda t: None if t is None else t.index_select(1, ret).contiguous()   # noqa: E731
    return pick(w.k), pick(w.v), pick(w.k_sz), pick(w.v_sz)


def empty_stream_cache(w: DecodeWorkload, sink_pages: int, ring_pages: int, fill_byte: int = 0xFF):
    """Tensors of a streaming-head cache for the workload's batch, every byte
    set to fill_byte: (k, v, k_sz, v_sz), pages [B][H_s][sink + ring] shaped
    like one (page, head) of the pool."""
    n_str = sum(1 for x in w.head_kind if x == 1)
    shape = (w.batch, n_str, sink_pages + ring_pages)
    k = torch.empty(shape + tuple(w.k.shape[2:]), dtype=w.k.dtype, device=w.k.device)
    v = torch.empty(shape + tuple(w.v.shape[2:]), dtype=w.v.dtype, device=w.v.device)
    k.view(torch.uint8).fill_(fill_byte)
    v.view(torch.uint8).fill_(fill_byte)
    k_sz = v_sz = None
    if w.k_sz is not None:
        k_sz = torch.empty(shape + (2,), dtype=torch.float16, device=w.k.device)
        v_sz = torch.empty_like(k_sz)
        k_sz.view(torch.uint8).fill_(fill_byte)
        v_sz.view(torch.uint8).fill_(fill_byte)
    return k, v, k_sz, v_sz


def token_rows(w: DecodeWorkload, step: int):
    """The K and V rows of the token each sequence appends at window step
    `step` (position ctx + step), every KV head, read out of the generated
    pool: ([B][H_kv][D], [B][H_kv][D]) in the pool dtype, or for int4 the codes
    ([B][H_kv][D/2] bytes, channel 2i in the low nibble) followed by the fp16
    (scale, zero) pairs of the token's page, ([B][H_kv][2], [B][H_kv][2])."""
    NP, D = w.page_size, w.head_dim
    bt = min(NP, 32)
    pos = torch.tensor([c + step for c in w.ctx], device=w.k.device)
    pages = w.page_table.long().gather(1, (pos // NP)[:, None])[:, 0]
    slot = pos % NP
    blk, r = slot // bt, slot % bt
    ks, vs = [], []
    for b in range(w.batch):
        kt = w.k[pages[b], :, blk[b], :, r[b], :]               # [H_kv][D/32][32 or 16 bytes]
        ks.append(kt.reshape(w.num_kv_heads, -1))
        if w.dtype == INT4:
            vb = w.v[pages[b], :, blk[b], :, r[b] // 2]          # [H_kv][D] bytes holding the token's nibble
            codes = (vb >> (4 * (int(r[b]) % 2))) & 15
            vs.append(codes[:, 0::2] | (codes[:, 1::2] << 4))
        else:
            vs.append(w.v[pages[b], :, blk[b], :, r[b]])          # [H_kv][D]
    k_new, v_new = torch.stack(ks).contiguous(), torch.stack(vs).contiguous()
    if w.dtype != INT4:
        return k_new, v_new
    return k_new, v_new, w.k_sz[pages].contiguous(), w.v_sz[pages].contiguous()
