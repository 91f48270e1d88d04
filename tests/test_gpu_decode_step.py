"""lsa_decode_step (append + select + attend in two launches: the selection
takes the newest token's key from the step's rows, the decode kernel attends
the token from its staged rows and writes it to its page) on a pool that holds
every head, against the fp64 oracle and against the three separate calls
(lsa_append_kv, lsa_select_pages, lsa_sparse_decode_attn).

The GPU pool starts as a copy of the generated one with every window token's
rows overwritten (NaN for f32 / bf16, code 15 for int4, and a zero (s, z)
pair for the int4 pages the window opens), so a step can only see its token,
and every later step the earlier tokens, through what the step itself wrote.
Bars: selections bit for bit, outputs within 1e-5 (f32) or 2e-2 (bf16, int4)
of the oracle; the pool bytes and statistics after the window equal those of
the three-call path byte for byte."""
import numpy as np
import pytest
import torch

import tests.helpers as H
import tests.test_gpu_decode as D
import tests.test_gpu_stats_select as S
from block_sparse_attention_logical_amd import lsa, workloads as W
from tests.test_gpu_stream_cache import wipe_window

pytestmark = pytest.mark.gpu
DEV = "cuda"


class StepRunner:
    """The decode window through lsa_decode_step (fused) or the three calls,
    on a wiped copy of the workload's every-head pool."""

    def __init__(self, w, fused, agg=lsa.AGG_SUM):
        self.w, self.fused = w, fused
        clone = lambda t: None if t is None else t.clone()  # noqa: E731
        self.k, self.v, self.k_sz, self.v_sz = clone(w.k), clone(w.v), clone(w.k_sz), clone(w.v_sz)
        wipe_window(w, self.k, self.v, self.k_sz, self.v_sz, slice(None))
        self.kv = lsa.KVPool(w.dtype, self.k, self.v, w.num_kv_heads, w.head_dim, w.page_size, w.logical_page,
                             w.num_pages, self.k_sz, self.v_sz)
        self.hd = H.heads(w, agg)
        lens0 = torch.tensor(w.ctx, dtype=torch.int32, device=DEV)
        self.stats = torch.zeros(lsa.page_stats_bytes(self.kv), dtype=torch.uint8, device=DEV)
        if max(w.ctx) > 0:
            lsa.build_page_stats(self.kv, w.page_table, lens0.clamp(min=1), self.stats, heads=self.hd)
        K = w.token_budget // w.page_size
        self.selected = torch.full((w.batch, w.num_kv_heads, K), -1, dtype=torch.int32, device=DEV)
        lens1 = lens0 + 1
        self.ws_step = torch.zeros(lsa.decode_step_workspace(self.kv, w.page_table, lens1, self.hd, w.token_budget),
                                   dtype=torch.uint8, device=DEV)
        self.ws_sel = torch.zeros(lsa.select_pages_workspace(self.kv, w.page_table, lens1, self.hd),
                                  dtype=torch.uint8, device=DEV)
        self.ws_dec = torch.zeros(lsa.decode_workspace(self.kv, w.page_table, lens1, self.hd, w.token_budget),
                                  dtype=torch.uint8, device=DEV)
        self.rows = [W.token_rows(w, i) for i in range(w.window)]
        self.history = []

    def step(self, i):
        w = self.w
        lens = w.seq_lens(i)
        rows = self.rows[i]
        out = torch.empty_like(w.q[i])
        if self.fused:
            lsa.decode_step(w.q[i], self.kv, w.page_table, lens, self.hd, rows[0], rows[1], self.stats,
                            w.token_budget, i, w.reuse_interval, self.selected, out, self.ws_step, *rows[2:])
        else:
            lsa.append_kv(self.kv, w.page_table, lens, self.hd, *rows, stats=self.stats)
            lsa.select_pages(w.q[i], self.kv, self.stats, w.page_table, lens, self.hd, w.token_budget, i,
                             w.reuse_interval, self.selected, self.ws_sel)
            lsa.sparse_decode_attn(w.q[i], self.kv, w.page_table, lens, self.hd, self.selected, w.token_budget,
                                   out, self.ws_dec)
        torch.cuda.synchronize()
        self.history.append(self.selected.cpu().numpy().copy())
        return out


def check_fused_window(w, agg=lsa.AGG_SUM, batches=None, kv_heads=None):
    """The fused window against the oracle (selections, outputs), then against
    the three-call window (selections, pool bytes, statistics)."""
    r = StepRunner(w, fused=True, agg=agg)
    gpu = [H.to_f64(r.step(i)) for i in range(w.window)]
    assert not any(np.isnan(g).any() for g in gpu)
    G = w.num_q_heads // w.num_kv_heads
    worst = excess = 0.0
    for b in (range(w.batch) if batches is None else batches):
        sel = {}
        ref = D.oracle_window(w, b, kv_heads=kv_heads, agg=agg, selections=sel)
        for (i, kv), expect in sel.items():
            assert np.array_equal(r.history[i][b, kv], expect), (b, i, kv, r.history[i][b, kv], expect)
        heads = range(w.num_q_heads) if kv_heads is None else [kv * G + h for kv in kv_heads for h in range(G)]
        for i in range(w.window):
            for h in heads:
                err = np.max(np.abs(gpu[i][b, h] - ref[i][h]))
                worst = max(worst, err)
                assert err <= D.tol(w), (b, i, h, err)
                if w.dtype != W.F32:
                    excess = max(excess, H.rounding_excess(gpu[i][b, h], ref[i][h]))
    if w.dtype != W.F32:
        print(f"{H.DTYPE_NAME[w.dtype]} decode step: max abs err {worst:.4f}, beyond the output's own rounding "
              f"{excess:.4f}")
        assert excess <= H.EXCESS_TOL, excess
    s3 = StepRunner(w, fused=False, agg=agg)
    for i in range(w.window):
        s3.step(i)
        assert np.array_equal(s3.history[i], r.history[i]), i
    for a, c in ((r.k, s3.k), (r.v, s3.v), (r.k_sz, s3.k_sz), (r.v_sz, s3.v_sz), (r.stats, s3.stats)):
        if a is not None:
            assert torch.equal(a.view(torch.uint8), c.view(torch.uint8))
    # the appends restored every wiped row: the pool is the generated one again
    assert torch.equal(r.k.view(torch.uint8), w.k.view(torch.uint8))
    assert torch.equal(r.v.view(torch.uint8), w.v.view(torch.uint8))
    return r, worst


CASES = [
    ("cfg1-f32", lambda: W.make_decode(1, DEV)),
    ("cfg2-bf16", lambda: W.make_decode(2, DEV, batch=3, ctx=[1000, 2500, 4096])),
    ("cfg2-bf16-page-edges", lambda: W.make_decode(2, DEV, batch=3, ctx=[63, 64, 65])),
    ("cfg5-int4", lambda: W.make_decode(5, DEV, batch=2, ctx=[127, 4096 + 17])),
    ("cfg5-int4-page-open", lambda: W.make_decode(5, DEV, batch=2, ctx=[2044, 1020], window=8)),
    ("cfg2-bf16-np16", lambda: W.make_decode(2, DEV, batch=2, ctx=[2000, 4105], window=8, page_size=16)),
    ("cfg5-int4-np16-nl8", lambda: W.make_decode(5, DEV, batch=2, ctx=[1999, 3000], window=8, page_size=16,
                                                 logical_page=8)),
    ("cfg4-bf16-np128", lambda: W.make_decode(4, DEV, batch=2, ctx=[5000, 9000], window=8)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_decode_step_window(name, make):
    w = make()
    r, worst = check_fused_window(w)
    print("max abs err", worst)
    S.check_stats(w, r.stats, [c + w.window for c in w.ctx], kinds=w.head_kind)


def test_decode_step_from_an_empty_sequence():
    """t = 0: the first step's only token is the one it appends."""
    w = W.make_decode(2, DEV, batch=2, ctx=[0, 0], window=3)
    check_fused_window(w)


@pytest.mark.parametrize("cfg", [2, 5])
def test_decode_step_max_aggregation(cfg):
    w = W.make_decode(cfg, DEV, batch=2, ctx=[6000, 9000], window=8)
    check_fused_window(w, agg=lsa.AGG_MAX)


@pytest.mark.parametrize("R", [1, 8])
def test_decode_step_reuse_interval(R):
    w = W.make_decode(2, DEV, batch=2, ctx=[3000, 4500], window=8)
    w.reuse_interval = R
    check_fused_window(w)


def test_decode_step_workspace_counters_return_to_zero():
    w = W.make_decode(5, DEV, batch=3, ctx=[700, 2100, 1500], window=4)
    r = StepRunner(w, fused=True)
    n = w.batch * w.num_kv_heads
    for i in range(w.window):
        r.step(i)
        assert int(r.ws_step[:4 * n].view(torch.int32).abs().sum()) == 0
