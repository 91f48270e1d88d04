"""GPU parity of the logical-page statistics and of page selection against the
fp64 oracle.  Statistics must match exactly (min / max involve no rounding);
selected page indices must match bit for bit, ties to the lower page."""
import numpy as np
import pytest
import torch

import oracle.lsa_oracle as O
import tests.helpers as H
from block_sparse_attention_logical_amd import lsa, workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def stats_view(w, stats):
    g = w.page_size // w.logical_page
    if w.dtype == W.INT4:
        return stats.view(torch.uint8).view(w.num_pages, w.num_kv_heads, g, w.head_dim)
    dt = torch.float32 if w.dtype == W.F32 else torch.bfloat16
    return stats.view(dt).view(w.num_pages, w.num_kv_heads, g, 2, w.head_dim)


def build_stats(w, lens, heads=None, first=None, max_new=0, stats=None):
    kv = H.kv_pool(w)
    if stats is None:
        stats = torch.full((lsa.page_stats_bytes(kv),), 0xAB, dtype=torch.uint8, device=DEV)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ft = None if first is None else torch.tensor(first, dtype=torch.int32, device=DEV)
    lsa.build_page_stats(kv, w.page_table, seq_lens, stats, heads=heads, first_token=ft, max_new_tokens=max_new)
    torch.cuda.synchronize()
    return stats


def gpu_page_stats(w, stats, b, kv, L):
    """GPU statistics of the logical pages of (b, kv) holding tokens < L."""
    g = w.page_size // w.logical_page
    n = -(-L // w.logical_page)
    j = torch.arange(n, device=DEV)
    pools = w.page_table[b].long()[j // g]
    sv = stats_view(w, stats)
    return sv[pools, kv, j % g].cpu()


def check_stats(w, stats, lens, kinds=None):
    for b, L in enumerate(lens):
        for kv in range(w.num_kv_heads):
            if kinds is not None and kinds[kv] != 0:
                continue
            got = gpu_page_stats(w, stats, b, kv, L)
            pool = H.seq_pool(w, b, kv, L)
            table = list(range(-(-L // w.page_size)))
            if w.dtype == W.INT4:
                cmin, cmax = O.page_code_stats(pool.k_codes(table, 0, L), w.logical_page)
                got = got.numpy()
                assert np.array_equal(got & 15, cmin), (b, kv)
                assert np.array_equal(got >> 4, cmax), (b, kv)
            else:
                kmin, kmax = O.page_stats(pool.keys(table, 0, L), w.logical_page)
                g64 = H.to_f64(got)
                assert np.array_equal(g64[:, 0], kmin), (b, kv)     # by value: signed zeros compare equal
                assert np.array_equal(g64[:, 1], kmax), (b, kv)


CASES = [
    ("cfg1-f32", lambda: W.make_decode(1, DEV)),
    ("cfg2-bf16-np16", lambda: W.make_decode(2, DEV, batch=2, ctx=[1000, 4100], page_size=16, logical_page=16)),
    ("cfg5-int4-np16-nl8", lambda: W.make_decode(5, DEV, batch=2, ctx=[2100, 5000], page_size=16, logical_page=8)),
    ("cfg2-bf16-small", lambda: W.make_decode(2, DEV, batch=3, ctx=[1000, 2500, 4096])),
    ("cfg4-bf16-np128-small", lambda: W.make_decode(4, DEV, batch=3, ctx=(1500, 6000))),
    ("cfg5-int4-small", lambda: W.make_decode(5, DEV, batch=2, ctx=[2100, 3333])),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_stats_full_build(name, make):
    w = make()
    lens = [c + w.window for c in w.ctx]
    stats = build_stats(w, lens)
    check_stats(w, stats, lens)


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_stats_incremental_update(name, make):
    """Build after the prompt, then update token by token (first_token = t)."""
    w = make()
    lens = list(w.ctx)
    stats = build_stats(w, lens)
    for i in range(w.window):
        first = [c + i for c in w.ctx]
        lens = [c + i + 1 for c in w.ctx]
        build_stats(w, lens, first=first, max_new=1, stats=stats)
    check_stats(w, stats, lens)


def test_stats_retrieval_heads_only():
    w = W.make_decode(2, DEV, batch=2, ctx=[700, 1300])
    lens = [c + 1 for c in w.ctx]
    stats = build_stats(w, lens, heads=H.heads(w))
    check_stats(w, stats, lens, kinds=w.head_kind)
    # streaming heads' statistics are left untouched
    sv = stats_view(w, stats).view(torch.uint8) if w.dtype != W.INT4 else stats_view(w, stats)
    for kv in range(w.num_kv_heads):
        if w.head_kind[kv]:
            assert bool((sv.reshape(w.num_pages, w.num_kv_heads, -1)[:, kv] == 0xAB).all())


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def run_select(w, step, lens, stats=None, selected=None, decode_step=0, agg=lsa.AGG_SUM):
    kv = H.kv_pool(w)
    hd = H.heads(w, agg)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    if stats is None:
        stats = build_stats(w, lens)
    K = w.token_budget // w.page_size
    if selected is None:
        selected = torch.full((w.batch, w.num_kv_heads, K), -7, dtype=torch.int32, device=DEV)
    ws = torch.zeros(lsa.select_pages_workspace(kv, w.page_table, seq_lens, hd), dtype=torch.uint8, device=DEV)
    lsa.select_pages(w.q[step], kv, stats, w.page_table, seq_lens, hd, w.token_budget, decode_step,
                     w.reuse_interval, selected, ws)
    torch.cuda.synchronize()
    return selected


def oracle_selection(w, step, b, kv, L, agg=lsa.AGG_SUM):
    G = w.num_q_heads // w.num_kv_heads
    keys, _ = H.seq_kv(w, b, kv, L)
    kmin, kmax = O.page_stats(keys, w.logical_page)
    q = H.to_f64(w.q[step, b, kv * G:(kv + 1) * G])
    S = O.logical_scores(q, kmin, kmax, H.AGG_NAME[agg])
    P = O.physical_scores(S, w.page_size // w.logical_page)
    K = w.token_budget // w.page_size
    return O.topk_pages(P, K), P


def check_selection(w, step, lens, selected, pairs=None, report=None, agg=lsa.AGG_SUM):
    K = w.token_budget // w.page_size
    sel = selected.cpu().numpy()
    for b, L in enumerate(lens):
        for kv in range(w.num_kv_heads):
            if w.head_kind[kv] != 0 or (pairs is not None and (b, kv) not in pairs):
                continue
            expect, P = oracle_selection(w, step, b, kv, L, agg)
            if report is not None and len(P) > K:
                s = np.sort(P)[::-1]
                report.append(abs(s[K - 1] - s[K]) / max(1.0, abs(s[K - 1])))
            assert np.array_equal(sel[b, kv], expect), (b, kv, sel[b, kv], expect)


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_select_matches_oracle(name, make):
    w = make()
    for step in range(min(2, w.window)):
        lens = [c + step + 1 for c in w.ctx]
        sel = run_select(w, step, lens)
        check_selection(w, step, lens, sel)
        # streaming heads' rows are not written
        for kv in range(w.num_kv_heads):
            if w.head_kind[kv]:
                assert bool((sel[:, kv] == -7).all())


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_select_max_aggregation_matches_oracle(name, make):
    """score_aggregation = LSA_AGG_MAX: the group's per-head page scores are
    combined by max; the selection still matches the oracle bit for bit."""
    w = make()
    lens = [c + 1 for c in w.ctx]
    sel = run_select(w, 0, lens, agg=lsa.AGG_MAX)
    check_selection(w, 0, lens, sel, agg=lsa.AGG_MAX)


def test_select_max_and_sum_aggregation_differ():
    """The two aggregations are different rankings on the bf16 workload (so the
    max-aggregation parity test above is not the sum test in disguise)."""
    w = W.make_decode(2, DEV, batch=2, ctx=[20000, 30000])      # 313 and 469 pages for K = 64
    lens = [c + 1 for c in w.ctx]
    a = run_select(w, 0, lens, agg=lsa.AGG_SUM).cpu().numpy()
    m = run_select(w, 0, lens, agg=lsa.AGG_MAX).cpu().numpy()
    ret = [kv for kv in range(w.num_kv_heads) if w.head_kind[kv] == 0]
    assert any(not np.array_equal(a[b, kv], m[b, kv]) for b in range(w.batch) for kv in ret)


def test_select_reuse_keeps_previous_selection():
    w = W.make_decode(2, DEV, batch=2, ctx=[3000, 5000])
    lens = [c + 1 for c in w.ctx]
    sel = run_select(w, 0, lens, decode_step=0)
    before = sel.clone()
    for step in (1, 2, 3):
        run_select(w, step, [c + step + 1 for c in w.ctx], selected=sel, decode_step=step)
        assert torch.equal(sel, before)
    run_select(w, 0, lens, selected=sel, decode_step=4)     # a multiple of R selects again
    check_selection(w, 0, lens, sel)


def test_select_short_sequences_pad_with_minus_one():
    """Fewer pages than the budget: every page, ascending, then -1."""
    w = W.make_decode(2, DEV, batch=3, ctx=[1, 64 * 5 - 1, 64 * 70])
    lens = [c + 1 for c in w.ctx]
    sel = run_select(w, 0, lens).cpu().numpy()
    K = w.token_budget // w.page_size
    for b, L in enumerate(lens):
        n = -(-L // w.page_size)
        for kv in range(w.num_kv_heads):
            if w.head_kind[kv] == 0 and n <= K:
                assert list(sel[b, kv]) == list(range(n)) + [-1] * (K - n)


def test_select_ties_go_to_lower_page():
    """Identical pages score identically; the lower page index wins."""
    w = W.make_decode(2, DEV, batch=1, ctx=[64 * 200 - 1])
    # copy page 7's keys over pages 100..199 of the sequence, and page 8's over 30..99
    tbl = w.page_table[0].long()
    w.k[tbl[7]] = (w.k[tbl[7]].float() * 3).to(w.k.dtype)      # make the copied page rank high
    for m in range(100, 200):
        w.k[tbl[m]] = w.k[tbl[7]]
    for m in range(30, 100):
        w.k[tbl[m]] = w.k[tbl[8]]
    lens = [w.ctx[0] + 1]
    sel = run_select(w, 0, lens)
    check_selection(w, 0, lens, sel)


def test_select_scores_current_page_from_keys():
    """Statistics built only up to the previous token: the logical page that
    holds the current token is scored from its keys, so the selection still
    matches the oracle (which sees every token)."""
    for cfg, kw in ((2, dict(batch=3, ctx=[1000, 2047, 5000])), (5, dict(batch=2, ctx=[777, 3000])),
                    (4, dict(batch=2, ctx=(3000, 6000))), (1, {})):
        w = W.make_decode(cfg, DEV, **kw)
        stats = build_stats(w, list(w.ctx))          # tokens < ctx only
        lens = [c + 1 for c in w.ctx]
        sel = run_select(w, 0, lens, stats=stats)
        check_selection(w, 0, lens, sel)


def test_select_full_size_cfg2():
    """Config 2 at full size (B = 8, 64K context): every retrieval head."""
    w = W.make_decode(2, DEV)
    lens = [c + 1 for c in w.ctx]
    sel = run_select(w, 0, lens)
    gaps = []
    check_selection(w, 0, lens, sel, report=gaps)
    print(f"smallest relative gap between the K-th and (K+1)-th page scores: {min(gaps):.3e}")


@pytest.mark.parametrize("cfg,pages,agg", [(2, 4096, lsa.AGG_SUM), (2, 4097, lsa.AGG_SUM), (5, 4096, lsa.AGG_SUM),
                                            (5, 4097, lsa.AGG_SUM), (2, 4096, lsa.AGG_MAX), (2, 4097, lsa.AGG_MAX)],
                         ids=["bf16-4096", "bf16-4097", "int4-4096", "int4-4097", "bf16-max-4096", "bf16-max-4097"])
def test_select_either_side_of_one_kernel_limit(cfg, pages, agg):
    """Up to 4096 pages per sequence the last score workgroup of a (sequence,
    head) runs its top-K; from 4097 pages a separate top-K kernel does.  Both
    sides of that limit, for the bf16 pool (config 2) with the group's scores
    summed and combined by max, and the int4 pool (config 5, whose 256K
    context has 4097 pages), with a shorter second sequence in the batch;
    every retrieval head, bit for bit."""
    w = W.make_decode(cfg, DEV, batch=2, ctx=[pages * 64 - 4, 3000])      # + 4 window tokens
    assert w.max_pages == pages
    lens = [c + 1 for c in w.ctx]
    sel = run_select(w, 0, lens, agg=agg)
    gaps = []
    check_selection(w, 0, lens, sel, report=gaps, agg=agg)
    print(f"smallest relative gap between the K-th and (K+1)-th page scores: {min(gaps):.3e}")
    del w
    torch.cuda.empty_cache()



@pytest.mark.parametrize("cfg,pages", [(2, 1025), (2, 2049), (5, 1025), (5, 2049)])
@pytest.mark.parametrize("mode", ["all-equal", "last-high", "random"])
def test_select_last_page_ranked_apart(cfg, pages, mode):
    """With the group's scores summed, the fused ranking holds 4 or 8 pages per
    thread of its 256 threads and ranks one more page apart, the last one
    (1025 or 2049 pages): it joins the K largest of the others when its
    score is above their K-th largest, and loses a tie to them.  Every key the
    same (all pages tie: pages 0 .. K-1 win), the last page's keys scaled up
    (it ranks first and takes the last slot), and the ordinary data; bit for
    bit against the oracle."""
    w = W.make_decode(cfg, DEV, batch=1, ctx=[pages * 64 - 4])
    lens = [w.ctx[0] + 1]
    n = -(-lens[0] // w.page_size)
    assert n == pages
    tbl = w.page_table[0, :n].long()
    if mode == "all-equal":
        if w.k_sz is None:
            w.k[tbl] = 1.0
        else:
            w.k[tbl] = 0x35
            w.k_sz[tbl] = w.k_sz[tbl[0]].clone()
    elif mode == "last-high":
        if w.k_sz is None:
            w.k[tbl[-1]] = (w.k[tbl[-1]].float() * 8).to(w.k.dtype)
        else:
            w.k_sz[tbl[-1], :, 0] *= 8
    sel = run_select(w, 0, lens)
    check_selection(w, 0, lens, sel)
    K = w.token_budget // w.page_size
    got = sel.cpu().numpy()
    for kv in range(w.num_kv_heads):
        if w.head_kind[kv] == 0:
            if mode == "all-equal":
                assert list(got[0, kv]) == list(range(K)), kv
            elif mode == "last-high":
                assert got[0, kv, K - 1] == n - 1, kv
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["wide-span", "zero-group", "ordinary"])
def test_select_int4_query_terms_and_the_integer_grid(mode):
    """int4 scoring takes a group's folded query terms (Qp, -Qn) as integers on
    one grid of 32 bits when they fit, which every generated query does
    ("ordinary"): then every score is exact.  A query whose terms span more
    than 32 bits ("wide-span": one channel of one head set to 2^-30, one of
    another group's to -1.25 * 2^-33) takes the fp64 products instead; a group
    whose query is all zero ("zero-group") scores every page 0 and keeps the
    lowest pages.  Each ranks as the oracle does.  (In the wide-span case
    neither side's fp64 sums need be exact; the K-th / (K+1)-th gap printed
    below is far above any rounding difference.)"""
    w = W.make_decode(5, DEV, batch=2, ctx=[6000, 9000])      # 94 and 141 pages for K = 64
    G = w.num_q_heads // w.num_kv_heads
    ret = [kv for kv in range(w.num_kv_heads) if w.head_kind[kv] == 0]
    if mode == "wide-span":
        w.q[0, 0, ret[0] * G, 5] = 2.0 ** -30
        w.q[0, 1, ret[1] * G + 1, 17] = -1.25 * 2.0 ** -33
    elif mode == "zero-group":
        w.q[0, 0, ret[0] * G:(ret[0] + 1) * G] = 0
    lens = [c + 1 for c in w.ctx]
    sel = run_select(w, 0, lens)
    gaps = []
    check_selection(w, 0, lens, sel, report=gaps)
    print("smallest relative K / K+1 gap", min(gaps))
    if mode == "zero-group":
        K = w.token_budget // w.page_size
        assert sel[0, ret[0]].cpu().tolist() == list(range(K))
