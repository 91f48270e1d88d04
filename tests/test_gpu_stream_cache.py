"""The constant-size streaming-head cache and the per-step append (a decode
step that appends its token, selects every R steps and attends, with the
streaming heads read from sink pages plus a ring of recent pages and the
retrieval heads from a pool that holds only them) against the fp64 oracle:
selections bit for bit, outputs within 1e-5 (f32) or 2e-2 (bf16, int4)."""
import numpy as np
import pytest
import torch

import oracle.lsa_oracle as O
import tests.helpers as H
import tests.test_gpu_decode as D
import tests.test_gpu_stats_select as S
from block_sparse_attention_logical_amd import lsa, workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def wipe_window(w, k, v, k_sz, v_sz, heads_of_pool):
    """Overwrite the window tokens' rows in a copy of the pool (NaN for f32 /
    bf16, code 15 for int4, the int4 (s, z) of pages the window opens), so
    that only the append can put them back."""
    NP, bt = w.page_size, min(w.page_size, 32)
    for b, c in enumerate(w.ctx):
        for i in range(w.window):
            t = c + i
            page = int(w.page_table[b, t // NP])
            s_ = t % NP
            blk, r = s_ // bt, s_ % bt
            if w.dtype == W.INT4:
                k[page, heads_of_pool, blk, :, r, :] = 0xFF
                v[page, heads_of_pool, blk, :, r // 2] |= 0xF << (4 * (r % 2))
                if s_ == 0:
                    k_sz[page, heads_of_pool] = 0
                    v_sz[page, heads_of_pool] = 0
            else:
                k[page, heads_of_pool, blk, :, r, :] = float("nan")
                v[page, heads_of_pool, blk, :, r] = float("nan")


class CacheRunner:
    """Decode through append + select + attend with the streaming heads in a
    stream cache filled from the prompt, the retrieval heads in a pool of their own."""

    def __init__(self, w, fused=False):
        self.w = w
        self.fused = fused
        full = H.kv_pool(w)
        self.hd = H.heads(w)
        sink, ring = lsa.stream_cache_pages(full, self.hd)
        self.sink, self.ring = sink, ring
        ck, cv, cks, cvs = W.empty_stream_cache(w, sink, ring)
        self.cache = lsa.StreamCache(sink, ring, ck, cv, cks, cvs)
        lens0 = torch.tensor(w.ctx, dtype=torch.int32, device=DEV)
        lsa.stream_cache_fill(full, w.page_table, lens0, self.hd, self.cache)
        self.wipe_cache_window(ck, cv, cks, cvs)
        k, v, k_sz, v_sz = W.retrieval_pool(w)
        wipe_window(w, k, v, k_sz, v_sz, slice(None))
        self.kv = lsa.KVPool(w.dtype, k, v, w.num_kv_heads, w.head_dim, w.page_size, w.logical_page, w.num_pages,
                             k_sz, v_sz, stream_cache=self.cache)
        self.stats = torch.zeros(lsa.page_stats_bytes(self.kv, self.hd), dtype=torch.uint8, device=DEV)
        lsa.build_page_stats(self.kv, w.page_table, lens0, self.stats, heads=self.hd)
        self.K = w.token_budget // w.page_size
        self.selected = torch.full((w.batch, w.num_kv_heads, self.K), -1, dtype=torch.int32, device=DEV)
        self.ws_sel = torch.zeros(lsa.select_pages_workspace(self.kv, w.page_table, lens0, self.hd),
                                  dtype=torch.uint8, device=DEV)
        self.ws_dec = torch.zeros(lsa.decode_workspace(self.kv, w.page_table, lens0, self.hd, w.token_budget),
                                  dtype=torch.uint8, device=DEV)
        self.ws_step = torch.zeros(lsa.decode_step_workspace(self.kv, w.page_table, lens0, self.hd, w.token_budget),
                                   dtype=torch.uint8, device=DEV)
        self.rows = [W.token_rows(w, i) for i in range(w.window)]
        self.history = []

    def wipe_cache_window(self, ck, cv, cks, cvs):
        """The filled cache pages copy whole pool pages, window tokens included:
        overwrite those rows of the prompt's last page so that only the append
        can put them back.  (A page the window opens takes the ring slot of a
        page that may still be read at the first window steps; that slot keeps
        the old page's rows until the append writes over them.)"""
        w = self.w
        NP, bt = w.page_size, min(w.page_size, 32)
        for b, c in enumerate(w.ctx):
            for i in range(w.window):
                t = c + i
                m, s_ = t // NP, t % NP
                if m != (c - 1) // NP:
                    continue
                cp = m if m < self.sink else self.sink + (m - self.sink) % self.ring
                blk, r = s_ // bt, s_ % bt
                if w.dtype == W.INT4:
                    ck[b, :, cp, blk, :, r, :] = 0xFF
                    cv[b, :, cp, blk, :, r // 2] |= 0xF << (4 * (r % 2))
                    if s_ == 0:
                        cks[b, :, cp] = 0
                        cvs[b, :, cp] = 0
                else:
                    ck[b, :, cp, blk, :, r, :] = float("nan")
                    cv[b, :, cp, blk, :, r] = float("nan")

    def step(self, i):
        w = self.w
        lens = w.seq_lens(i)
        if self.fused:
            out = torch.empty_like(w.q[i])
            rows = self.rows[i]
            lsa.decode_step(w.q[i], self.kv, w.page_table, lens, self.hd, rows[0], rows[1], self.stats,
                            w.token_budget, i, w.reuse_interval, self.selected, out, self.ws_step,
                            *rows[2:])
            torch.cuda.synchronize()
            self.history.append(self.selected.cpu().numpy().copy())
            return out
        lsa.append_kv(self.kv, w.page_table, lens, self.hd, *self.rows[i], stats=self.stats)
        lsa.select_pages(w.q[i], self.kv, self.stats, w.page_table, lens, self.hd, w.token_budget, i,
                         w.reuse_interval, self.selected, self.ws_sel)
        out = torch.empty_like(w.q[i])
        lsa.sparse_decode_attn(w.q[i], self.kv, w.page_table, lens, self.hd, self.selected, w.token_budget, out,
                               self.ws_dec)
        torch.cuda.synchronize()
        self.history.append(self.selected.cpu().numpy().copy())
        return out


def check_cache_window(w, batches=None, kv_heads=None, fused=False):
    r = CacheRunner(w, fused=fused)
    gpu = [H.to_f64(r.step(i)) for i in range(w.window)]
    assert not any(np.isnan(g).any() for g in gpu)
    worst = 0.0
    G = w.num_q_heads // w.num_kv_heads
    for b in (range(w.batch) if batches is None else batches):
        sel = {}
        ref = D.oracle_window(w, b, kv_heads=kv_heads, selections=sel)
        for (i, kv), expect in sel.items():
            assert np.array_equal(r.history[i][b, kv], expect), (b, i, kv)
        heads = range(w.num_q_heads) if kv_heads is None else [kv * G + h for kv in kv_heads for h in range(G)]
        for i in range(w.window):
            for h in heads:
                err = np.max(np.abs(gpu[i][b, h] - ref[i][h]))
                worst = max(worst, err)
                assert err <= D.tol(w), (b, i, h, err)
    return r, worst


def stats_as_full_layout(w, r):
    """The retrieval-only statistics pool scattered into the every-head layout
    that the statistics checks read."""
    ret = [h for h in range(w.num_kv_heads) if w.head_kind[h] == 0]
    g = w.page_size // w.logical_page
    per = r.stats.numel() // (w.num_pages * len(ret) * g)
    full = torch.zeros((w.num_pages, w.num_kv_heads, g, per), dtype=torch.uint8, device=DEV)
    full[:, ret] = r.stats.view(w.num_pages, len(ret), g, per)
    return full.reshape(-1)


CASES = [
    ("cfg2-bf16", lambda: W.make_decode(2, DEV, batch=3, ctx=[3000, 4501, 6000], window=8)),
    ("cfg5-int4", lambda: W.make_decode(5, DEV, batch=2, ctx=[2047, 5001], window=8)),
    ("cfg1-f32", lambda: W.make_decode(1, DEV, window=16)),
    ("cfg2-bf16-np16", lambda: W.make_decode(2, DEV, batch=2, ctx=[2000, 4105], window=8, page_size=16)),
    ("cfg5-int4-np16", lambda: W.make_decode(5, DEV, batch=2, ctx=[1999, 3000], window=8, page_size=16)),
]


@pytest.mark.parametrize("fused", [False, True], ids=["3calls", "fused"])
@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_append_select_attend_window_with_stream_cache(name, make, fused):
    """The whole window through append + select + attend (three calls, or
    lsa_decode_step's two launches): selections and outputs match the oracle
    (which reads every token of every head), and the statistics the appends
    updated equal the oracle's at the final length."""
    w = make()
    r, worst = check_cache_window(w, fused=fused)
    print("max abs err", worst)
    S.check_stats(w, stats_as_full_layout(w, r), [c + w.window for c in w.ctx], kinds=w.head_kind)


def test_stream_cache_fill_copies_sink_and_recent_pages():
    """After the fill at the prompt's length, cache page j of (b, s) holds the
    pool page the mapping assigns it (sink pages, then ring slot (m - sink) %
    ring of the ring_pages most recent pages), byte for byte; pages past the
    sequence keep their previous bytes."""
    w = W.make_decode(2, DEV, batch=3, ctx=[100, 1000, 5000], page_size=64)
    full, hd = H.kv_pool(w), H.heads(w)
    sink, ring = lsa.stream_cache_pages(full, hd)
    assert (sink, ring) == (1, 17)                    # 64 sink tokens, 1024 local tokens, 64-token pages
    ck, cv, cks, cvs = W.empty_stream_cache(w, sink, ring, fill_byte=0x5A)
    cache = lsa.StreamCache(sink, ring, ck, cv, cks, cvs)
    lens = torch.tensor(w.ctx, dtype=torch.int32, device=DEV)
    lsa.stream_cache_fill(full, w.page_table, lens, hd, cache)
    torch.cuda.synchronize()
    st = [h for h in range(w.num_kv_heads) if w.head_kind[h] == 1]
    for b, L in enumerate(w.ctx):
        m_cur = (L - 1) // w.page_size
        expect = {}
        for m in range(m_cur + 1):
            if m < sink:
                expect[m] = m
            elif m > m_cur - ring:
                expect[sink + (m - sink) % ring] = m
        for s, kvh in enumerate(st):
            for cp in range(sink + ring):
                if cp in expect:
                    page = int(w.page_table[b, expect[cp]])
                    assert torch.equal(ck[b, s, cp].view(torch.uint8), w.k[page, kvh].view(torch.uint8)), (b, s, cp)
                    assert torch.equal(cv[b, s, cp].view(torch.uint8), w.v[page, kvh].view(torch.uint8)), (b, s, cp)
                else:
                    assert bool((ck[b, s, cp].view(torch.uint8) == 0x5A).all()), (b, s, cp)
