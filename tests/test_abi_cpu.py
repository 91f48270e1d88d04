"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, sizes its buffers as documented, and rejects invalid
arguments with the documented status before launching anything.  No call
here reaches a kernel launch (each either fails validation or takes a
documented no-launch path), so no GPU is needed."""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_attention_logical_amd import lsa, workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")

FAKE = 0x10000          # a non-NULL device address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lsa.LIB_PATH):
        from block_sparse_attention_logical_amd import build
        build.build(verbose=False)
    return lsa.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:lsa_status|const char \*)\s*(lsa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_entry_points():
    names = header_functions()
    for n in ("lsa_build_page_stats", "lsa_select_pages", "lsa_sparse_decode_attn", "lsa_sparse_prefill_attn"):
        assert n in names
    assert set(names) == set(lsa.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lsa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    defined = set(re.findall(r"\sT\s(lsa_\w+)$", out, flags=re.M))
    for name in header_functions():
        assert name in defined, name
        assert hasattr(lib, name)


def test_version(lib):
    assert lsa.version().startswith("lsa ") and "gfx950" in lsa.version()


def test_version_names_the_sources_of_this_tree(lib):
    """The loaded library was built from the sources in this tree: its version
    carries their hash (a stale build fails here)."""
    from block_sparse_attention_logical_amd import build
    assert lsa.version().endswith("src " + build.source_sha())


def kv_desc(dtype=lsa.BF16, heads=8, D=128, NP=64, NL=16, P=100, sz=False):
    k_sz = FAKE if sz else None
    return lsa.LsaKV(dtype, heads, D, NP, NL, 0, P, FAKE, FAKE, k_sz, k_sz)


def seqs_desc(B=2, max_pages=10):
    return lsa.LsaSeqs(B, max_pages, FAKE, FAKE)


def heads_desc(kinds=(0, 1, 0, 1, 0, 1, 0, 1), hq=32, sink=64, local=1024, sb=1, lb=16):
    buf = (ctypes.c_uint8 * len(kinds))(*kinds)
    h = lsa.LsaHeads(ctypes.cast(buf, ctypes.c_void_p), hq, sink, local, sb, lb)
    h._keep = buf
    return h


def stats_bytes(lib, kv):
    out = ctypes.c_size_t(0)
    st = lib.lsa_page_stats_bytes(ctypes.byref(kv), None, ctypes.byref(out))
    return st, out.value


def test_stats_bytes_sizes(lib):
    assert stats_bytes(lib, kv_desc(lsa.BF16, 8, 128, 64, 16, 100)) == (0, 100 * 8 * 4 * 2 * 128 * 2)
    assert stats_bytes(lib, kv_desc(lsa.F32, 2, 64, 64, 16, 17)) == (0, 17 * 2 * 4 * 2 * 64 * 4)
    assert stats_bytes(lib, kv_desc(lsa.INT4, 8, 128, 128, 16, 10, sz=True)) == (0, 10 * 8 * 8 * 128)


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), lsa.LSA_ERR_UNSUPPORTED),
    (dict(NP=48, NL=16), lsa.LSA_ERR_UNSUPPORTED),      # 3 logical pages: not a power of two
    (dict(NP=64, NL=24), lsa.LSA_ERR_UNSUPPORTED),
    (dict(NP=40, NL=8), lsa.LSA_ERR_UNSUPPORTED),       # not a power of two
    (dict(NP=96, NL=32), lsa.LSA_ERR_UNSUPPORTED),
    (dict(NP=16, NL=32), lsa.LSA_ERR_INVALID_ARG),      # logical page longer than the page
    (dict(NP=8, NL=16), lsa.LSA_ERR_INVALID_ARG),
    (dict(heads=0), lsa.LSA_ERR_UNSUPPORTED),
    (dict(heads=65), lsa.LSA_ERR_UNSUPPORTED),
    (dict(P=0), lsa.LSA_ERR_INVALID_ARG),
    (dict(dtype=7), lsa.LSA_ERR_INVALID_ARG),
    (dict(dtype=lsa.INT4), lsa.LSA_ERR_INVALID_ARG),    # int4 without scale / zero arrays
    (dict(dtype=lsa.BF16, sz=True), lsa.LSA_ERR_INVALID_ARG),
])
def test_kv_validation(lib, kw, code):
    st, _ = stats_bytes(lib, kv_desc(**kw))
    assert st == code
    assert lsa.last_error() != ""


def test_null_descriptor_and_reserved(lib):
    out = ctypes.c_size_t(0)
    assert lib.lsa_page_stats_bytes(None, None, ctypes.byref(out)) == lsa.LSA_ERR_INVALID_ARG
    kv = kv_desc()
    kv.reserved = 1
    assert stats_bytes(lib, kv)[0] == lsa.LSA_ERR_INVALID_ARG


def select(lib, kv=None, seqs=None, heads=None, q_dtype=lsa.BF16, budget=4096, step=0, R=4, ws_bytes=1 << 30,
           selected=FAKE, q=FAKE, stats=FAKE):
    kv = kv or kv_desc()
    seqs = seqs or seqs_desc()
    heads = heads or heads_desc()
    return lib.lsa_select_pages(q, q_dtype, ctypes.byref(kv), stats, ctypes.byref(seqs), ctypes.byref(heads),
                                budget, step, R, selected, FAKE, ws_bytes, None)


def test_select_validation(lib):
    assert select(lib, budget=4000) == lsa.LSA_ERR_INVALID_ARG       # not a multiple of N_P
    assert select(lib, budget=32) == lsa.LSA_ERR_INVALID_ARG         # below one page
    assert select(lib, R=0) == lsa.LSA_ERR_INVALID_ARG
    assert select(lib, step=-1) == lsa.LSA_ERR_INVALID_ARG
    assert select(lib, q_dtype=lsa.INT4) == lsa.LSA_ERR_INVALID_ARG
    assert select(lib, ws_bytes=16) == lsa.LSA_ERR_WORKSPACE
    assert select(lib, selected=None) == lsa.LSA_ERR_INVALID_ARG
    assert select(lib, heads=heads_desc(hq=30)) == lsa.LSA_ERR_INVALID_ARG
    assert select(lib, heads=heads_desc(hq=8 * 17)) == lsa.LSA_ERR_UNSUPPORTED
    assert select(lib, heads=heads_desc(kinds=(0, 1, 2, 1, 0, 1, 0, 1))) == lsa.LSA_ERR_INVALID_ARG
    assert select(lib, heads=heads_desc(local=0)) == lsa.LSA_ERR_INVALID_ARG
    bad_agg = heads_desc()
    bad_agg.score_aggregation = 2
    assert select(lib, heads=bad_agg) == lsa.LSA_ERR_INVALID_ARG
    assert select(lib, seqs=seqs_desc(max_pages=0)) == lsa.LSA_ERR_UNSUPPORTED
    assert select(lib, seqs=seqs_desc(max_pages=16385)) == lsa.LSA_ERR_UNSUPPORTED   # above the top-K limit
    assert select(lib, seqs=lsa.LsaSeqs(2, 10, None, FAKE)) == lsa.LSA_ERR_INVALID_ARG


def test_select_reuse_step_is_a_no_op(lib):
    # steps that are not multiples of the reuse interval keep the previous
    # selection: the call succeeds without launching anything
    for step in (1, 2, 3, 5, 7):
        assert select(lib, step=step, R=4) == lsa.LSA_OK
    # no retrieval head: nothing to select
    assert select(lib, step=0, heads=heads_desc(kinds=(1,) * 8)) == lsa.LSA_OK


def test_select_workspace_size(lib):
    out = ctypes.c_size_t(0)
    st = lib.lsa_select_pages_workspace(ctypes.byref(kv_desc()), ctypes.byref(seqs_desc(8, 1025)),
                                        ctypes.byref(heads_desc()), ctypes.byref(out))
    # B * H_kv int32 arrival counters (padded to 256 bytes), then one fp64
    # score per physical page of every (sequence, KV head)
    assert st == 0 and out.value == 256 + 8 * 8 * 1025 * 8


def decode(lib, kv=None, heads=None, q_dtype=lsa.BF16, selected=FAKE, ws_bytes=1 << 30, scale=0.0, batch=2):
    kv = kv or kv_desc()
    heads = heads or heads_desc()
    return lib.lsa_sparse_decode_attn(FAKE, q_dtype, ctypes.byref(kv), ctypes.byref(seqs_desc(batch)),
                                      ctypes.byref(heads), selected, 4096, scale, FAKE, None, FAKE, ws_bytes, None)


def test_decode_validation(lib):
    assert decode(lib, q_dtype=lsa.F32) == lsa.LSA_ERR_UNSUPPORTED            # f32 q with bf16 pool
    assert decode(lib, selected=None) == lsa.LSA_ERR_INVALID_ARG
    assert decode(lib, ws_bytes=64) == lsa.LSA_ERR_WORKSPACE
    assert decode(lib, scale=-1.0) == lsa.LSA_ERR_INVALID_ARG
    assert decode(lib, scale=float("nan")) == lsa.LSA_ERR_INVALID_ARG
    # all heads streaming: selected may be NULL; batch 0 launches nothing
    assert decode(lib, heads=heads_desc(kinds=(1,) * 8), selected=None, batch=0) == lsa.LSA_OK


def test_decode_workspace_size(lib):
    # records of 32 + G*D floats per chunk, after one int32 counter per
    # (sequence, KV head).  65 retrieval pages and 1 + 15 + 2 = 18 streaming
    # pages per (sequence, head), chunks of at most 8 pages (four wavefronts of
    # 128 tokens), and 2 x 256 workgroup slots for the bf16 kernel.
    def ws(batch):
        out = ctypes.c_size_t(0)
        st = lib.lsa_decode_workspace(ctypes.byref(kv_desc()), ctypes.byref(seqs_desc(batch, 1025)),
                                      ctypes.byref(heads_desc()), 4096, ctypes.byref(out))
        assert st == 0
        return out.value
    # B = 16: 16 x (4 x 9 + 4 x 3) = 768 workgroups of 8 pages, more than the slots: 9 chunks
    assert ws(16) == 512 + 16 * 8 * 9 * (32 + 4 * 128) * 4
    # B = 8: 384 workgroups of 8 pages fit; 6 pages per chunk is the smallest size that still
    # fits (8 x (4 x 11 + 4 x 3) = 448; 5 pages: 544): 11 chunks per retrieval head
    assert ws(8) == 256 + 8 * 8 * 11 * (32 + 4 * 128) * 4


def prefill(lib, kv=None, q_dtype=lsa.BF16, block=64, T=1000):
    kv = kv or kv_desc()
    return lib.lsa_sparse_prefill_attn(FAKE, q_dtype, ctypes.byref(kv), FAKE, T, ctypes.byref(heads_desc()),
                                       block, 0.0, FAKE, None, None)


def test_prefill_validation(lib):
    assert prefill(lib, block=32) == lsa.LSA_ERR_UNSUPPORTED
    assert prefill(lib, kv=kv_desc(NP=32)) == lsa.LSA_ERR_UNSUPPORTED
    assert prefill(lib, kv=kv_desc(dtype=lsa.F32)) == lsa.LSA_ERR_UNSUPPORTED  # f32 path is head_dim 64
    assert prefill(lib, q_dtype=lsa.F32) == lsa.LSA_ERR_UNSUPPORTED            # mixed pair
    assert prefill(lib, T=-1) == lsa.LSA_ERR_INVALID_ARG
    assert prefill(lib, T=0) == lsa.LSA_OK                                     # nothing to do


def prefill_csr(lib, kv=None, block=64, T=1000, rp=FAKE, ci=FAKE, nnz=10, hq=32):
    kv = kv or kv_desc()
    return lib.lsa_sparse_prefill_attn_csr(FAKE, lsa.BF16, ctypes.byref(kv), FAKE, T, hq, block, rp, ci, nnz,
                                           None, 0.0, FAKE, None, None)


def test_prefill_csr_validation(lib):
    assert prefill_csr(lib, block=128) == lsa.LSA_ERR_UNSUPPORTED
    assert prefill_csr(lib, rp=None) == lsa.LSA_ERR_INVALID_ARG
    assert prefill_csr(lib, ci=None) == lsa.LSA_ERR_INVALID_ARG
    assert prefill_csr(lib, nnz=-1) == lsa.LSA_ERR_INVALID_ARG
    assert prefill_csr(lib, hq=12) == lsa.LSA_ERR_INVALID_ARG                 # not a multiple of 8 KV heads
    assert prefill_csr(lib, hq=8 * 32) == lsa.LSA_ERR_UNSUPPORTED             # group of 32
    assert prefill_csr(lib, T=0) == lsa.LSA_OK                                # nothing to do
    assert prefill_csr(lib, T=0, ci=None, nnz=0) == lsa.LSA_OK


def test_check_block_mask():
    """The host-side mask checker accepts CSR lists built from tile masks and
    names the first malformed row."""
    m = W.random_tile_masks(2, 9, 0.4, 3)
    rp, ci = W.csr_from_tile_masks(m)
    lsa.check_block_mask(rp, ci, 2, 9 * 64)
    lsa.check_block_mask(rp, ci, 2, 8 * 64 + 1)                 # ragged last tile
    empty_rows = m.clone()
    empty_rows[1, 4] = False
    lsa.check_block_mask(*W.csr_from_tile_masks(empty_rows), 2, 9 * 64)   # empty rows are allowed
    bad = ci.clone()
    bad[int(rp[0, 5])] = 6                                       # tile above the diagonal
    with pytest.raises(lsa.LsaError, match="query tile 5"):
        lsa.check_block_mask(rp, bad, 2, 9 * 64)
    r2 = int(rp[1, 6])
    assert int(rp[1, 7]) - r2 >= 2
    bad = ci.clone()
    bad[r2], bad[r2 + 1] = ci[r2 + 1], ci[r2]                    # descending within a row
    with pytest.raises(lsa.LsaError, match="ascending"):
        lsa.check_block_mask(rp, bad, 2, 9 * 64)
    bad_rp = rp.clone()
    bad_rp[0, 3] = bad_rp[0, 2] - 1                              # offsets decrease
    with pytest.raises(lsa.LsaError, match="head 0"):
        lsa.check_block_mask(bad_rp, ci, 2, 9 * 64)
    bad_rp = rp.clone()
    bad_rp[1, 9] = ci.numel() + 1                                # past nnz
    with pytest.raises(lsa.LsaError, match="head 1"):
        lsa.check_block_mask(bad_rp, ci, 2, 9 * 64)


def test_block_mask_schedule():
    """The work order of a mask lists every (KV head, query tile, head group)
    item once.  At group sizes above 2 rows come in non-increasing length; at
    1 and 2, where a bf16 work item takes 4 / G query tiles
    n-1-QT*j-QT+1 .. n-1-QT*j, each group's highest tile comes first, ordered
    by the longest row of its group, then every other code by its own row."""
    for H, G, n in ((8, 4, 13), (4, 8, 9), (32, 1, 5), (4, 1, 11), (8, 2, 7)):
        m = W.random_tile_masks(H, n, 0.35, seed=H * n)
        m[0, 2] = False                                          # an empty row
        rp, _ = W.csr_from_tile_masks(m)
        order = lsa.block_mask_schedule(rp, H, H * G, n * 64 - 3)
        hg = -(-G // 4)
        assert sorted(order.tolist()) == list(range(H * n * hg))
        lens = (rp[:, 1:] - rp[:, :-1]).reshape(-1)             # [H * n], row (kv, a) at kv * n + a
        qt = 4 // G if G <= 2 else 1
        is_lead = [(n - 1 - (int(c) // hg) % n) % qt == 0 for c in order]
        n_lead = H * (-(-n // qt)) * hg
        assert all(is_lead[:n_lead]) and not any(is_lead[n_lead:])

        def group_len(c):
            kv, a = divmod(int(c) // hg, n)
            return max(int(lens[kv * n + a - s]) for s in range(qt) if a - s >= 0)
        key = [group_len(c) for c in order[:n_lead]] + [int(lens[int(c) // hg]) for c in order[n_lead:]]
        for part in (key[:n_lead], key[n_lead:]):
            assert all(x >= y for x, y in zip(part, part[1:]))
    with pytest.raises(lsa.LsaError):
        lsa.block_mask_schedule(rp, 32, 31, 5 * 64)


def test_stats_validation(lib):
    kv = kv_desc()
    seqs = seqs_desc()
    assert lib.lsa_build_page_stats(ctypes.byref(kv), ctypes.byref(seqs), None, None, 0, None, None) == \
        lsa.LSA_ERR_INVALID_ARG
    assert lib.lsa_build_page_stats(ctypes.byref(kv), ctypes.byref(seqs), None, None, -1, FAKE, None) == \
        lsa.LSA_ERR_INVALID_ARG
    # empty batch: nothing to build
    assert lib.lsa_build_page_stats(ctypes.byref(kv), ctypes.byref(seqs_desc(0)), None, None, 0, FAKE, None) == 0


def test_decode_noalloc_validation(lib):
    """The static-scratch decode call validates like lsa_sparse_decode_attn and
    rejects a batch whose scratch exceeds its 16 MiB array before touching the
    device."""
    def call(B=2, q_dtype=lsa.BF16, selected=FAKE, budget=4096, heads=None):
        return lib.lsa_sparse_decode_attn_noalloc(FAKE, q_dtype, ctypes.byref(kv_desc()),
                                                  ctypes.byref(seqs_desc(B, 1025)),
                                                  ctypes.byref(heads or heads_desc()), selected, budget, 0.0,
                                                  FAKE, None, None)
    assert call(q_dtype=lsa.F32) == lsa.LSA_ERR_UNSUPPORTED
    assert call(selected=None) == lsa.LSA_ERR_INVALID_ARG
    # 8 x 8 heads at a 4096-token budget need 1.25 MB; 128 sequences need 20 MB
    assert call(B=128) == lsa.LSA_ERR_UNSUPPORTED
    assert "16777216-byte static scratch" in lsa.last_error()
    assert call(B=0) == lsa.LSA_OK                      # an empty batch launches nothing


@pytest.mark.parametrize("NP,NL", [(16, 16), (16, 8), (32, 16), (256, 16)])
def test_kv_page_sizes_accepted(lib, NP, NL):
    """16-token pages (one 16-token layout block) and 32..256-token pages."""
    st, nbytes = stats_bytes(lib, kv_desc(NP=NP, NL=NL))
    assert st == lsa.LSA_OK
    assert nbytes == 100 * 8 * (NP // NL) * 2 * 128 * 2


def test_stream_cache_pages_follow_the_lambda_window_only(lib):
    """The streaming-head cache needs ceil(sink / N_P) sink pages and
    ceil(local / N_P) + 1 ring pages, whatever the context length."""
    kv = kv_desc(NP=64, NL=16)
    sink, ring = ctypes.c_int32(0), ctypes.c_int32(0)
    for local, expect in ((1024, 17), (2048, 33), (1, 2), (64, 2), (65, 3)):
        st = lib.lsa_stream_cache_pages(ctypes.byref(kv), ctypes.byref(heads_desc(sink=64, local=local)),
                                        ctypes.byref(sink), ctypes.byref(ring))
        assert st == lsa.LSA_OK and (sink.value, ring.value) == (1, expect)
    st = lib.lsa_stream_cache_pages(ctypes.byref(kv_desc(NP=16, NL=16)), ctypes.byref(heads_desc(sink=64, local=1024)),
                                    ctypes.byref(sink), ctypes.byref(ring))
    assert st == lsa.LSA_OK and (sink.value, ring.value) == (4, 65)


def test_stream_cache_validation(lib):
    """A pool with a stream cache needs the head classification, a cache
    large enough for the Lambda window, and no prefill."""
    kv = kv_desc()
    small = lsa.LsaStreamCache(1, 16, FAKE, FAKE, None, None)      # ring 16 < ceil(1024 / 64) + 1
    kv.stream_cache = ctypes.cast(ctypes.pointer(small), ctypes.c_void_p)
    out = ctypes.c_size_t(0)
    assert lib.lsa_page_stats_bytes(ctypes.byref(kv), None, ctypes.byref(out)) == lsa.LSA_ERR_INVALID_ARG
    assert lib.lsa_page_stats_bytes(ctypes.byref(kv), ctypes.byref(heads_desc()), ctypes.byref(out)) == \
        lsa.LSA_ERR_INVALID_ARG
    good = lsa.LsaStreamCache(1, 17, FAKE, FAKE, None, None)
    kv.stream_cache = ctypes.cast(ctypes.pointer(good), ctypes.c_void_p)
    assert lib.lsa_page_stats_bytes(ctypes.byref(kv), ctypes.byref(heads_desc()), ctypes.byref(out)) == lsa.LSA_OK
    assert out.value == 100 * 4 * 4 * 2 * 128 * 2        # four retrieval heads in the pool
    assert lib.lsa_sparse_prefill_attn(FAKE, lsa.BF16, ctypes.byref(kv), FAKE, 1000, ctypes.byref(heads_desc()),
                                       64, 0.0, FAKE, None, None) == lsa.LSA_ERR_UNSUPPORTED
    # an int4 cache needs its scale / zero arrays, a bf16 one must not have them
    bad = lsa.LsaStreamCache(1, 17, FAKE, FAKE, FAKE, FAKE)
    kv.stream_cache = ctypes.cast(ctypes.pointer(bad), ctypes.c_void_p)
    assert lib.lsa_page_stats_bytes(ctypes.byref(kv), ctypes.byref(heads_desc()), ctypes.byref(out)) == \
        lsa.LSA_ERR_INVALID_ARG


def test_decode_step_validation(lib):
    """lsa_decode_step rejects bad arguments of any of its three parts before
    it launches anything (the fake device addresses are never touched)."""
    kv, h, seqs = kv_desc(), heads_desc(), seqs_desc()
    need = ctypes.c_size_t(0)
    assert lib.lsa_decode_step_workspace(ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(h), 4096,
                                         ctypes.byref(need)) == lsa.LSA_OK
    sel, dec = ctypes.c_size_t(0), ctypes.c_size_t(0)
    lib.lsa_select_pages_workspace(ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(h), ctypes.byref(sel))
    lib.lsa_decode_workspace(ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(h), 4096, ctypes.byref(dec))
    assert need.value == max(sel.value, dec.value) > 0

    def call(kvd=kv, hd=h, q_dtype=lsa.BF16, k_new=FAKE, sz=None, stats=FAKE, budget=4096, step=0, R=4,
             selected=FAKE, scale=0.0, out=FAKE, ws_bytes=None):
        return lib.lsa_decode_step(FAKE, q_dtype, ctypes.byref(kvd), ctypes.byref(seqs), ctypes.byref(hd), k_new,
                                   FAKE, sz, sz, stats, budget, step, R, selected, scale, out, FAKE,
                                   need.value if ws_bytes is None else ws_bytes, None)

    assert call(k_new=None) == lsa.LSA_ERR_INVALID_ARG
    assert call(sz=FAKE) == lsa.LSA_ERR_INVALID_ARG                  # (s, z) rows for a bf16 pool
    assert call(kvd=kv_desc(dtype=lsa.INT4, sz=True)) == lsa.LSA_ERR_INVALID_ARG   # int4 without them
    assert call(stats=None) == lsa.LSA_ERR_INVALID_ARG               # retrieval heads need statistics
    assert call(selected=None) == lsa.LSA_ERR_INVALID_ARG
    assert call(ws_bytes=need.value - 1) == lsa.LSA_ERR_WORKSPACE
    assert call(budget=100) == lsa.LSA_ERR_INVALID_ARG
    assert call(R=0) == lsa.LSA_ERR_INVALID_ARG
    assert call(step=-1) == lsa.LSA_ERR_INVALID_ARG
    assert call(out=None) == lsa.LSA_ERR_INVALID_ARG                 # a decode-only check, still before any launch
    assert call(scale=float("nan")) == lsa.LSA_ERR_INVALID_ARG
    assert call(q_dtype=lsa.F32) == lsa.LSA_ERR_UNSUPPORTED          # f32 queries on a bf16 pool
    # reuse steps skip the selection, not the checks
    assert call(step=1, out=None) == lsa.LSA_ERR_INVALID_ARG


def test_append_validation(lib):
    kv = kv_desc()
    h = heads_desc()
    seqs = seqs_desc()
    assert lib.lsa_append_kv(ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(h), None, FAKE, None, None, None,
                             None) == lsa.LSA_ERR_INVALID_ARG
    assert lib.lsa_append_kv(ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(h), FAKE, FAKE, FAKE, FAKE, None,
                             None) == lsa.LSA_ERR_INVALID_ARG       # (s, z) rows for a bf16 pool
    kv4 = kv_desc(dtype=lsa.INT4, sz=True)
    assert lib.lsa_append_kv(ctypes.byref(kv4), ctypes.byref(seqs), ctypes.byref(h), FAKE, FAKE, None, None, None,
                             None) == lsa.LSA_ERR_INVALID_ARG       # int4 without (s, z) rows
    assert lib.lsa_append_kv(ctypes.byref(kv), ctypes.byref(seqs), None, FAKE, FAKE, None, None, None,
                             None) == lsa.LSA_ERR_INVALID_ARG       # heads are required
