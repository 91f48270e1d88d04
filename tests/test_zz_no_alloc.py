"""The decode entry point that allocates nothing (lsa_sparse_decode_attn_noalloc,
its scratch in the library's static per-GPU array) against
lsa_sparse_decode_attn with a caller workspace: the same outputs and the same
refreshed statistics, bit for bit, on two calls in a row, the second with a
smaller batch and shorter contexts (the array keeps the first call's
contents)."""
import pytest
import torch

import tests.helpers as H
from block_sparse_attention_logical_amd import lsa, workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def prepared(w):
    """Statistics built after the prompt and a selection for window step 0."""
    kv, hd = H.kv_pool(w), H.heads(w)
    lens0 = torch.tensor(w.ctx, dtype=torch.int32, device=DEV)
    stats = torch.zeros(lsa.page_stats_bytes(kv), dtype=torch.uint8, device=DEV)
    lsa.build_page_stats(kv, w.page_table, lens0, stats, heads=hd)
    K = w.token_budget // w.page_size
    sel = torch.full((w.batch, w.num_kv_heads, K), -1, dtype=torch.int32, device=DEV)
    lens = w.seq_lens(0)
    ws = torch.zeros(lsa.select_pages_workspace(kv, w.page_table, lens, hd), dtype=torch.uint8, device=DEV)
    lsa.select_pages(w.q[0], kv, stats, w.page_table, lens, hd, w.token_budget, 0, w.reuse_interval, sel, ws)
    return kv, hd, lens, stats, sel


def compare_one_call(w):
    kv, hd, lens, stats, sel = prepared(w)
    stats_a, stats_b = stats.clone(), stats.clone()
    ref = torch.empty_like(w.q[0])
    ws = torch.zeros(lsa.decode_workspace(kv, w.page_table, lens, hd, w.token_budget), dtype=torch.uint8,
                     device=DEV)
    lsa.sparse_decode_attn(w.q[0], kv, w.page_table, lens, hd, sel, w.token_budget, ref, ws, stats=stats_a)
    got = torch.full_like(w.q[0], float("nan"))
    lsa.sparse_decode_attn_noalloc(w.q[0], kv, w.page_table, lens, hd, sel, w.token_budget, got, stats=stats_b)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(stats_a, stats_b)


@pytest.mark.parametrize("cfg", [2, 5, 1])
def test_noalloc_decode_matches_workspace_call_twice(cfg):
    if cfg == 1:
        first, second = W.make_decode(1, DEV), W.make_decode(1, DEV, ctx=[300], window=2)
    else:
        first = W.make_decode(cfg, DEV, batch=4, ctx=[3000, 9000, 4500, 6100])
        second = W.make_decode(cfg, DEV, batch=2, ctx=[700, 2100], seed=cfg + 100)
    compare_one_call(first)
    compare_one_call(second)


def test_noalloc_decode_in_hip_graph():
    """Captured in a HIP graph (the callers it is for) and replayed twice with
    eager work between the replays: bitwise the eager call's outputs."""
    w = W.make_decode(2, DEV, batch=3, ctx=[3000, 4500, 6000])
    kv, hd, lens, stats, sel = prepared(w)
    eager = torch.empty_like(w.q[0])
    lsa.sparse_decode_attn_noalloc(w.q[0], kv, w.page_table, lens, hd, sel, w.token_budget, eager)
    torch.cuda.synchronize()
    out = torch.empty_like(w.q[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lsa.sparse_decode_attn_noalloc(w.q[0], kv, w.page_table, lens, hd, sel, w.token_budget, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lsa.sparse_decode_attn_noalloc(w.q[0], kv, w.page_table, lens, hd, sel, w.token_budget, out)
    for rep in range(2):
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
        del junk


def test_noalloc_decode_rejects_oversized_batch():
    """A batch whose scratch exceeds the 16 MiB array is refused on the host."""
    w = W.make_decode(2, DEV, batch=2, ctx=[1000, 2000])
    kv, hd = H.kv_pool(w), H.heads(w)
    big_table = torch.zeros((128, w.max_pages), dtype=torch.int32, device=DEV)
    big_lens = torch.full((128,), 1000, dtype=torch.int32, device=DEV)
    sel = torch.zeros((128, w.num_kv_heads, w.token_budget // w.page_size), dtype=torch.int32, device=DEV)
    out = torch.empty((128, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros_like(out)
    with pytest.raises(lsa.LsaError) as e:
        lsa.sparse_decode_attn_noalloc(q, kv, big_table, big_lens, hd, sel, w.token_budget, out)
    assert e.value.status == lsa.LSA_ERR_UNSUPPORTED
