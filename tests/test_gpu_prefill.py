"""GPU parity of block-sparse prefill attention against the fp64 oracle, and
the tile counter against the oracle's block accounting."""
import json
import os

import numpy as np
import pytest
import torch

import oracle.lsa_oracle as O
import tests.helpers as H
from block_sparse_attention_logical_amd import lsa, workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_prefill(p, counter=True):
    kv = lsa.KVPool(p.dtype, p.k, p.v, p.num_kv_heads, p.head_dim, p.page_size, p.logical_page, p.num_pages)
    hd = lsa.Heads(p.head_kind, p.num_q_heads, 0, 1, p.sink_blocks, p.local_blocks)
    out = torch.full_like(p.q, float("nan"))
    cnt = torch.zeros(1, dtype=torch.int64, device=DEV) if counter else None
    lsa.sparse_prefill_attn(p.q, kv, p.page_table, p.seq_len, hd, out, tile_counter=cnt)
    torch.cuda.synchronize()
    return out, (int(cnt.item()) if counter else None)


def seq_kv(p, kv):
    """Keys and values [T][D] float64 of one KV head, through the page table."""
    n = p.page_table.numel()
    rows = p.page_table.long()
    pool = O.Pool(H.DTYPE_NAME[p.dtype], H.bits(p.k[rows, kv][:, None]), H.bits(p.v[rows, kv][:, None]),
                  p.page_size, p.head_dim)
    table = list(range(n))
    return pool.keys(table, 0, p.seq_len), pool.values(table, 0, p.seq_len)


def expected_tiles(p):
    n = -(-p.seq_len // 64)
    G = p.num_q_heads // p.num_kv_heads
    return sum(G * O.block_counts(n, p.head_kind[kv], p.sink_blocks, p.local_blocks)[0]
               for kv in range(p.num_kv_heads))


def check(p, out, rows=None, heads=None, tol=2e-2):
    G = p.num_q_heads // p.num_kv_heads
    got = H.to_f64(out)
    worst = excess = 0.0
    for kv in range(p.num_kv_heads):
        hs = [kv * G + h for h in range(G)]
        if heads is not None:
            hs = [h for h in hs if h in heads]
        if not hs:
            continue
        keys, values = seq_kv(p, kv)
        for h in hs:
            q = H.to_f64(p.q[:, h])
            ref = O.prefill_attention(q, keys, values, p.head_kind[kv], 64, p.sink_blocks, p.local_blocks,
                                      1 / np.sqrt(p.head_dim), rows=rows)
            g = got[:, h] if rows is None else got[rows, h]
            err = np.max(np.abs(g - ref))
            worst = max(worst, err)
            assert err <= tol, (kv, h, err)
            if p.dtype == W.BF16:
                excess = max(excess, H.rounding_excess(g, ref))
    if p.dtype == W.BF16:
        print(f"bf16 prefill: max abs err {worst:.4f}, beyond the output's own rounding {excess:.4f}")
        assert excess <= H.EXCESS_TOL, excess
    return worst


def test_prefill_cfg1_f32():
    p = W.make_prefill(1, DEV)
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p)
    print("max abs err", check(p, out, tol=1e-5))


@pytest.mark.parametrize("T", [777, 64, 1, 1088])
def test_prefill_cfg3_small(T):
    p = W.make_prefill(3, DEV, seq_len=T)
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p)
    print("max abs err", check(p, out))


def test_prefill_all_retrieval_and_all_streaming():
    for kinds in ([0] * 8, [1] * 8):
        p = W.make_prefill(3, DEV, seq_len=1500, head_kind=kinds)
        out, cnt = run_prefill(p)
        assert cnt == expected_tiles(p)
        check(p, out, heads=[0, 5, 13, 31])


def test_prefill_deterministic():
    p = W.make_prefill(3, DEV, seq_len=700)
    a, _ = run_prefill(p)
    b, _ = run_prefill(p)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefill_full_size_cfg3_sampled():
    """Config 3 at full size (T = 131072, 32 heads): every output is written
    (no NaN left), the tile counter equals the oracle's 34,125,696 non-empty
    (head, tile) pairs, and sampled rows of one retrieval and one streaming
    head match the oracle."""
    p = W.make_prefill(3, DEV)
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p) == 34125696
    assert not bool(torch.isnan(out).any())
    ret = [kv for kv in range(8) if p.head_kind[kv] == 0][0]
    st = [kv for kv in range(8) if p.head_kind[kv] == 1][0]
    rows = [0, 1, 63, 64, 1000, 1023, 1024, 1087, 65536, 100000, 131071]
    print("max abs err", check(p, out, rows=rows, heads=[ret * 4 + 1, st * 4 + 2]))


@pytest.mark.parametrize("T", [777, 1088, 64, 200])
def test_prefill_cfg7_mha_small(T):
    """Multi-head attention (32 KV heads, group size 1)."""
    p = W.make_prefill(7, DEV, seq_len=T)
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p)
    print("max abs err", check(p, out, heads=[0, 1, 7, 18, 31]))


@pytest.mark.parametrize("T", [777, 1088, 64, 130])
def test_prefill_group2_small(T):
    """Two query heads per KV head (32 / 16 heads): a workgroup takes two query tiles."""
    p = W.make_prefill(3, DEV, seq_len=T, num_kv_heads=16)
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p)
    print("max abs err", check(p, out, heads=[0, 1, 6, 17, 30, 31]))


@pytest.mark.parametrize("D,NP,H_kv,T", [(64, 64, 8, 777), (64, 128, 8, 1088), (64, 64, 32, 700),
                                         (64, 256, 16, 1300), (128, 256, 8, 1000), (128, 128, 32, 900)])
def test_prefill_head_dim_and_page_size(D, NP, H_kv, T):
    """head_dim 64 and 128 with pages of 1 to 4 tiles, for one, two and four
    query tiles per workgroup (group sizes 4, 2 and 1)."""
    p = W.make_prefill(3, DEV, seq_len=T, head_dim=D, page_size=NP, num_kv_heads=H_kv)
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p)
    G = p.num_q_heads // p.num_kv_heads
    print("max abs err", check(p, out, heads=[0, G - 1, 13, 31]))


@pytest.mark.parametrize("H_q,H_kv,T", [(24, 8, 777), (40, 8, 1088), (64, 8, 700), (32, 2, 900)])
def test_prefill_group_sizes(H_q, H_kv, T):
    """Group sizes 3, 5, 8 and 16: several workgroups per (KV head, query
    tile), the last one with fewer than four heads."""
    p = W.make_prefill(3, DEV, seq_len=T, num_q_heads=H_q, num_kv_heads=H_kv)
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p)
    G = H_q // H_kv
    print("max abs err", check(p, out, heads=sorted({0, 3, G - 1, G, H_q - 1})))


def test_prefill_full_size_cfg7_mha_sampled():
    """Config 7 at full size (T = 131072, 32 query and 32 KV heads, 16 of them
    streaming): the same 34,125,696 non-empty (head, tile) pairs as the
    grouped layer, no NaN left, sampled rows of one retrieval and one
    streaming head against the oracle."""
    p = W.make_prefill(7, DEV)
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p) == 34125696
    assert not bool(torch.isnan(out).any())
    ret = [kv for kv in range(32) if p.head_kind[kv] == 0][0]
    st = [kv for kv in range(32) if p.head_kind[kv] == 1][0]
    rows = [0, 63, 64, 1087, 65536, 131071]
    print("max abs err", check(p, out, rows=rows, heads=[ret, st]))
    del out, p
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# static block masks (CSR)
# ---------------------------------------------------------------------------

def run_prefill_csr(p, masks, scheduled=True):
    """masks: [H_kv][n][n] bool tile masks; returns (out, tile counter).  The
    work order of the mask is used unless scheduled is False."""
    kv = lsa.KVPool(p.dtype, p.k, p.v, p.num_kv_heads, p.head_dim, p.page_size, p.logical_page, p.num_pages)
    row_ptr, col_idx = W.csr_from_tile_masks(masks)
    lsa.check_block_mask(row_ptr, col_idx, p.num_kv_heads, p.seq_len)
    order = lsa.block_mask_schedule(row_ptr, p.num_kv_heads, p.num_q_heads, p.seq_len).to(DEV) if scheduled else None
    out = torch.full_like(p.q, float("nan"))
    cnt = torch.zeros(1, dtype=torch.int64, device=DEV)
    lsa.sparse_prefill_attn_csr(p.q, kv, p.page_table, p.seq_len, p.num_q_heads, row_ptr.to(DEV),
                                col_idx.to(DEV), out, order=order, tile_counter=cnt)
    torch.cuda.synchronize()
    return out, int(cnt.item())


def check_mask(p, out, masks, heads=None, rows=None, tol=2e-2):
    G = p.num_q_heads // p.num_kv_heads
    got = H.to_f64(out)
    worst = excess = 0.0
    for kv in range(p.num_kv_heads):
        hs = [kv * G + h for h in range(G) if heads is None or kv * G + h in heads]
        if not hs:
            continue
        keys, values = seq_kv(p, kv)
        m = np.asarray(masks[kv], dtype=bool)
        for h in hs:
            ref = O.block_mask_attention(H.to_f64(p.q[:, h]), keys, values, m, 64, 1 / np.sqrt(p.head_dim), rows=rows)
            g = got[:, h] if rows is None else got[rows, h]
            err = np.max(np.abs(g - ref))
            worst = max(worst, err)
            assert err <= tol, (kv, h, err)
            if p.dtype == W.BF16:
                excess = max(excess, H.rounding_excess(g, ref))
    if p.dtype == W.BF16:
        print(f"bf16 prefill: max abs err {worst:.4f}, beyond the output's own rounding {excess:.4f}")
        assert excess <= H.EXCESS_TOL, excess
    return worst


@pytest.mark.parametrize("cfg,T,heads,scheduled,H_kv,D", [(1, 1024, None, True, None, None),
                                                          (3, 777, [0, 5, 13, 22, 31], True, None, None),
                                                          (3, 1088, [2, 9, 27], False, None, None),
                                                          (7, 777, [0, 1, 14, 31], True, None, None),
                                                          (7, 1088, [0, 3, 30, 31], False, None, None),
                                                          (3, 900, [0, 1, 6, 29, 30, 31], True, 16, None),
                                                          (3, 700, [0, 1, 17, 31], False, 16, None),
                                                          (7, 1000, [0, 2, 29, 31], True, None, 64),
                                                          (3, 830, [0, 1, 14, 31], True, 16, 64)])
def test_prefill_csr_random_masks(cfg, T, heads, scheduled, H_kv, D):
    """Random static masks (30% of the tiles below the diagonal, the diagonal
    kept except in one head, so some query tiles have no key tiles), with and
    without the mask's work order, at head_dim 128 and 64; at group sizes 1
    and 2 a workgroup walks the union of 4 / G query tiles' rows."""
    p = W.make_prefill(cfg, DEV, seq_len=T, num_kv_heads=H_kv, head_dim=D)
    n = -(-T // 64)
    masks = W.random_tile_masks(p.num_kv_heads, n, 0.3, seed=cfg * 1000 + T)
    masks[-1] = W.random_tile_masks(1, n, 0.3, seed=T, diagonal=False)[0]
    out, cnt = run_prefill_csr(p, masks, scheduled)
    G = p.num_q_heads // p.num_kv_heads
    assert cnt == G * int(masks.sum())
    tol = 1e-5 if p.dtype == W.F32 else 2e-2
    print("max abs err", check_mask(p, out, masks, heads=heads, tol=tol))


def test_prefill_csr_golden_10_of_21():
    """The pages' worked example on the GPU: a 6 x 6 tile grid with 10 of its 21
    causal tiles kept, for every KV head; the tile counter counts 10 tiles per
    query head and the outputs match the oracle."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "block_mask_10_of_21.json")) as f:
        g = json.load(f)
    n = g["n_blocks"]
    gm = torch.zeros((n, n), dtype=torch.bool)
    for a, c in g["nonempty"]:
        gm[a, c] = True
    p = W.make_prefill(3, DEV, seq_len=n * 64)
    masks = gm[None].expand(p.num_kv_heads, n, n).clone()
    out, cnt = run_prefill_csr(p, masks)
    assert cnt == g["expected_nonempty"] * p.num_q_heads
    print("max abs err", check_mask(p, out, masks))


def test_prefill_csr_kind_masks_equal_analytic():
    """The causal and Lambda patterns given as CSR lists give bitwise the
    outputs and the tile count of the head-kind call."""
    for cfg, T in ((3, 1500), (7, 1100), (1, 1024)):
        p = W.make_prefill(cfg, DEV, seq_len=T)
        n = -(-T // 64)
        masks = torch.stack([torch.from_numpy(O.kind_tile_mask(n, p.head_kind[kv], p.sink_blocks, p.local_blocks))
                             for kv in range(p.num_kv_heads)])
        a, ca = run_prefill(p)
        b, cb = run_prefill_csr(p, masks)
        assert ca == cb == expected_tiles(p)
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), cfg


@pytest.mark.parametrize("n,H_q", [(4096, 4), (4097, 4), (4096, 8)])
def test_prefill_csr_either_side_of_union_limit(n, H_q):
    """At group sizes 1 and 2 a bf16 workgroup walks the union of 4 / G query
    tiles' rows for up to 4096 tiles (the LDS tile list full at n = 4096) and
    takes one query tile past it (n = 4097).  With causal and Lambda heads
    given as CSR lists and the mask's work order, the counter and the outputs
    equal the head-kind call's bitwise, and sampled rows of a causal head
    match the oracle."""
    T = 64 * n - 5
    p = W.make_prefill(7, DEV, seq_len=T, num_q_heads=H_q, num_kv_heads=4, head_kind=[0, 1, 1, 0])
    masks = torch.stack([torch.from_numpy(O.kind_tile_mask(n, p.head_kind[kv], p.sink_blocks, p.local_blocks))
                         for kv in range(p.num_kv_heads)])
    b, cb = run_prefill_csr(p, masks)
    del masks
    a, ca = run_prefill(p)
    assert cb == ca == expected_tiles(p)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    print("max abs err", check(p, b, rows=[0, 64 * 4095 + 3, T - 1], heads=[H_q - 1]))
    del a, b, p
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [3, 7])
def test_prefill_csr_full_size(cfg):
    """Full-size prefill (T = 131072) with its head-kind patterns given as CSR
    lists and the mask's work order (config 3: GQA 4; config 7: MHA, where a
    workgroup walks the union of four query tiles' rows): the counter gives
    34,125,696 as for the head-kind call, and the outputs equal that call's
    bitwise."""
    p = W.make_prefill(cfg, DEV)
    n = -(-p.seq_len // 64)
    masks = torch.stack([torch.from_numpy(O.kind_tile_mask(n, p.head_kind[kv], p.sink_blocks, p.local_blocks))
                         for kv in range(p.num_kv_heads)])
    b, cb = run_prefill_csr(p, masks)
    del masks
    a, ca = run_prefill(p)
    assert cb == ca == 34125696
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    del a, b, p
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [1, 3])
def test_prefill_ignores_slots_past_the_sequence(cfg):
    """The last page's slots past the sequence (tokens 1000..1023) hold NaN in
    K and V (f32 NaN, or bf16 0x7FC0): no query reads them, so the outputs have
    no NaN and match the oracle, including the rows of the ragged last tile."""
    p = W.make_prefill(cfg, DEV, seq_len=1000)
    last = int(p.page_table[-1])
    for s_ in range(p.seq_len % p.page_size, p.page_size):
        blk, r = s_ // 32, s_ % 32              # key tiles [blk][D/32][32][32], value rows [blk][D][32]
        p.k[last, :, blk, :, r, :] = float("nan")
        p.v[last, :, blk, :, r] = float("nan")
    out, cnt = run_prefill(p)
    assert cnt == expected_tiles(p)
    assert not torch.isnan(out.float()).any()
    heads = None if cfg == 1 else {0, 5, 17, 31}
    print("max abs err", check(p, out, heads=heads, tol=1e-5 if cfg == 1 else 2e-2))
