"""Plain, slow fp64 CPU oracle for unified block-sparse attention with
hierarchical, query-aware KV page selection.

THIS MODULE IS TEST INFRASTRUCTURE.  Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it.  The GPU library never calls
it, and it shares no code, header, table or helper with the GPU library.

Sources (cited by page title and section):

  [LS-X] "MLSys 2025論文解説: LServe — 統一疎アテンションによる長文脈LLM推論の効率化"
         (explainer of LServe, MLSys 2025), section 技術的詳細 with its
         subsections 静的スパーシティ (streaming heads, Lambda mask),
         動的スパーシティ (page score equation S^j), 階層的ページング
         (logical vs physical pages, max reduction), 統一ブロックスパース
         アテンション (mermaid figure; block sparsity speed-up 1/(1-r) with the
         10-of-21 example) and Reusable Page Selection (reuse for k = 4 steps).
  [LS-A] "LServe: Efficient Long-sequence LLM Serving with Unified Sparse
         Attention" (abstract page): half the heads become streaming heads; a
         constant number of KV pages suffices regardless of context length.

Where the pages leave a step open, the reading taken is stated at the function
that takes it (readings Z1..Z27, listed together in the design notes of the
repository).

Data conventions (the layout of the caller-owned paged KV pool; a page is
N_P/BT blocks of BT = min(N_P, 32) consecutive tokens):
  * K  (f32 / bf16): [P][H_kv][N_P/BT][D/32][BT][32]   key (p, c) of a page at
                     [p // BT][c // 32][p % BT][c % 32]
  * V  (f32 / bf16): [P][H_kv][N_P/BT][D][BT]          value (p, c) at
                     [p // BT][c][p % BT]
  * K  (int4):       [P][H_kv][N_P/BT][D/32][BT][16] u8, the K tiles with
                     channels 2i, 2i+1 of a row in byte i (2i in the low nibble)
  * V  (int4):       [P][H_kv][N_P/BT][D][BT/2] u8, the V rows with tokens 2j,
                     2j+1 in byte j (2j in the low nibble)
  * k_sz, v_sz:      [P][H_kv][2] fp16 bits   (scale s, zero z); x = (c - z) * s
  * bf16 arrays are passed as uint16 bit patterns, fp16 as uint16 bit patterns.
Token p of sequence b lives in pool page page_table[b][p // N_P], slot p % N_P.

Everything is computed in float64.  No blocking, fusion or reordering beyond
what the definitions state.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

RETRIEVAL = 0
STREAMING = 1


# ---------------------------------------------------------------------------
# O1: exact conversion of stored values to float64
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exact (bf16 is the top half
    of an IEEE binary32)."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, exact."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Split bytes into 4-bit codes along the last axis: byte b holds element
    2i in its low nibble and element 2i+1 in its high nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & np.uint8(0x0F)
    hi = packed >> np.uint8(4)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant_int4(codes: np.ndarray, scale: float, zero: float) -> np.ndarray:
    """KV4 dequantisation x = (c - z) * s, in float64 (the quantised-KV
    co-design that [LS-X] pairs with the sparse path; per page and KV head
    scale and zero point, reading Z17)."""
    return (np.asarray(codes, dtype=np.float64) - zero) * scale


@dataclass
class Pool:
    """Host copy of a paged KV pool (see the module docstring for layout)."""
    dtype: str                    # "f32" | "bf16" | "int4"
    k: np.ndarray                 # raw storage, layout as documented above
    v: np.ndarray
    page_size: int                # N_P
    head_dim: int                 # D
    k_sz: Optional[np.ndarray] = None   # [P][H_kv][2] uint16 (fp16 bits)
    v_sz: Optional[np.ndarray] = None

    def _untile_k(self, a: np.ndarray) -> np.ndarray:
        """[N_P/BT][D/32][BT][32] key tiles of one page -> [N_P][D]."""
        bt = min(self.page_size, 32)
        a = np.asarray(a).reshape(self.page_size // bt, self.head_dim // 32, bt, 32)
        return a.transpose(0, 2, 1, 3).reshape(self.page_size, self.head_dim)

    def _untile_v(self, a: np.ndarray) -> np.ndarray:
        """[N_P/BT][D][BT] value rows of one page -> [N_P][D]."""
        bt = min(self.page_size, 32)
        a = np.asarray(a).reshape(self.page_size // bt, self.head_dim, bt)
        return a.transpose(0, 2, 1).reshape(self.page_size, self.head_dim)

    def _page_codes_k(self, page: int, kv: int) -> np.ndarray:
        """INT4: the key codes of one (pool page, KV head) as [N_P][D] uint8."""
        return self._untile_k(unpack_int4(self.k[page, kv]))

    def _page_rows_k(self, page: int, kv: int) -> np.ndarray:
        """All N_P keys of one (pool page, KV head) as [N_P][D] float64."""
        if self.dtype == "f32":
            return self._untile_k(np.asarray(self.k[page, kv], dtype=np.float64))
        if self.dtype == "bf16":
            return self._untile_k(bf16_bits_to_f64(self.k[page, kv]))
        s, z = fp16_bits_to_f64(self.k_sz[page, kv])
        return dequant_int4(self._page_codes_k(page, kv), s, z)

    def _page_rows_v(self, page: int, kv: int) -> np.ndarray:
        """All N_P values of one (pool page, KV head) as [N_P][D] float64."""
        if self.dtype == "f32":
            return self._untile_v(np.asarray(self.v[page, kv], dtype=np.float64))
        if self.dtype == "bf16":
            return self._untile_v(bf16_bits_to_f64(self.v[page, kv]))
        codes = self._untile_v(unpack_int4(self.v[page, kv]))     # [N_P][D]
        s, z = fp16_bits_to_f64(self.v_sz[page, kv])
        return dequant_int4(codes, s, z)

    def k_codes(self, page_table_row: Sequence[int], kv: int, length: int) -> np.ndarray:
        """INT4 only: the raw key codes of tokens 0..length-1, [length][D] uint8."""
        assert self.dtype == "int4"
        rows = []
        for m in range(-(-length // self.page_size)):
            rows.append(self._page_codes_k(int(page_table_row[m]), kv))
        return np.concatenate(rows, axis=0)[:length] if rows else np.zeros((0, self.head_dim), np.uint8)

    def keys(self, page_table_row: Sequence[int], kv: int, length: int) -> np.ndarray:
        """Keys of tokens 0..length-1 of one sequence and KV head, [length][D]
        float64.  Token p sits in pool page page_table_row[p // N_P]."""
        rows = [self._page_rows_k(int(page_table_row[m]), kv)
                for m in range(-(-length // self.page_size))]
        if not rows:
            return np.zeros((0, self.head_dim))
        return np.concatenate(rows, axis=0)[:length]

    def values(self, page_table_row: Sequence[int], kv: int, length: int) -> np.ndarray:
        rows = [self._page_rows_v(int(page_table_row[m]), kv)
                for m in range(-(-length // self.page_size))]
        if not rows:
            return np.zeros((0, self.head_dim))
        return np.concatenate(rows, axis=0)[:length]


# ---------------------------------------------------------------------------
# O2: logical-page channel statistics   ([LS-X] 動的スパーシティ, 階層的ページング)
# ---------------------------------------------------------------------------

def logical_page_count(length: int, logical_page: int) -> int:
    """Number of logical pages that hold at least one valid token (Z7)."""
    return -(-length // logical_page)


def page_stats(keys: np.ndarray, logical_page: int):
    """Channel-wise min and max of the keys of every logical page.

    keys: [L][D] (valid tokens only).  Logical page j covers tokens
    [j*N_L, min((j+1)*N_L, L)); pages with no token are not produced (Z7).
    Returns (kmin, kmax), each [ceil(L/N_L)][D].
    """
    L, D = keys.shape
    n = logical_page_count(L, logical_page)
    kmin = np.empty((n, D))
    kmax = np.empty((n, D))
    for j in range(n):
        block = keys[j * logical_page: min((j + 1) * logical_page, L)]
        kmin[j] = np.min(block, axis=0)
        kmax[j] = np.max(block, axis=0)
    return kmin, kmax


def page_code_stats(codes: np.ndarray, logical_page: int):
    """INT4 variant: min and max of the 4-bit codes per logical page and
    channel.  For s > 0 dequantisation is increasing, so these are the codes
    of the dequantised keys' min and max (reading Z17)."""
    L, D = codes.shape
    n = logical_page_count(L, logical_page)
    cmin = np.empty((n, D), dtype=np.uint8)
    cmax = np.empty((n, D), dtype=np.uint8)
    for j in range(n):
        block = codes[j * logical_page: min((j + 1) * logical_page, L)]
        cmin[j] = np.min(block, axis=0)
        cmax[j] = np.max(block, axis=0)
    return cmin, cmax


# ---------------------------------------------------------------------------
# O3: query-aware logical-page score       ([LS-X] 動的スパーシティ, the S^j equation)
# ---------------------------------------------------------------------------

SUM, MAX = "sum", "max"


def logical_scores(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray, aggregation: str = SUM) -> np.ndarray:
    """S^j of every logical page for one GQA group.

    For one query head h the score is the equation of [LS-X] as printed,
    S_h^j = sum over channels i of max(q_h[i] * kmax^j[i], q_h[i] * kmin^j[i]).
    The heads of a group share one selection; their scores are combined by
    `aggregation`: "sum" adds them (reading Z1, the default), "max" takes the
    largest.  With G = 1 both are the printed equation.

    q_group: [G][D] float64, the query heads that share one KV head.
    kmin, kmax: [n][D].  Returns [n] float64.
    """
    q = np.asarray(q_group, dtype=np.float64)
    n = kmin.shape[0]
    per_head = np.zeros((q.shape[0], n))
    for h in range(q.shape[0]):
        a = q[h][None, :] * kmax          # [n][D]
        b = q[h][None, :] * kmin
        per_head[h] = np.sum(np.maximum(a, b), axis=1)
    if aggregation == SUM:
        return per_head.sum(axis=0)
    if aggregation == MAX:
        return per_head.max(axis=0)
    raise ValueError(f"unknown aggregation {aggregation!r}")


# ---------------------------------------------------------------------------
# O4: physical page importance = max over its logical pages   ([LS-X] 階層的ページング)
# ---------------------------------------------------------------------------

def physical_scores(logical: np.ndarray, g: int) -> np.ndarray:
    """P_m = max{S^j : j // g == m} over the logical pages that exist
    (N_P = g * N_L).  Returns [ceil(n/g)]."""
    n = logical.shape[0]
    m_count = -(-n // g)
    out = np.empty(m_count)
    for m in range(m_count):
        out[m] = np.max(logical[m * g: min((m + 1) * g, n)])
    return out


# ---------------------------------------------------------------------------
# O5: top-K physical pages, ties to the lower sequence page index
#     ([LS-X] mermaid figure "Top-K物理ページ"; [LS-A] constant page budget)
# ---------------------------------------------------------------------------

def topk_pages(phys: np.ndarray, k: int) -> np.ndarray:
    """The k pages of largest score, ties broken towards the lower sequence
    page index m (Z5); emitted in ascending m and padded with -1 (Z6)."""
    n = phys.shape[0]
    order = sorted(range(n), key=lambda m: (-float(phys[m]), m))
    chosen = sorted(order[:k])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(chosen)] = chosen
    return out


def select_pages(q_group, kmin, kmax, g: int, k: int, aggregation: str = SUM) -> np.ndarray:
    """O3 -> O4 -> O5 for one (sequence, retrieval KV head)."""
    return topk_pages(physical_scores(logical_scores(q_group, kmin, kmax, aggregation), g), k)


# ---------------------------------------------------------------------------
# O7: attended key set of the decode token   ([LS-X] 静的スパーシティ, mermaid figure)
# ---------------------------------------------------------------------------

def attended_retrieval(t: int, selected: np.ndarray, page_size: int) -> np.ndarray:
    """Keys p <= t whose physical page is selected or is the current page
    floor(t / N_P) (reading Z10).  Returns a boolean mask of length t+1."""
    pages = set(int(m) for m in selected if m >= 0)
    pages.add(t // page_size)
    return np.array([(p // page_size) in pages for p in range(t + 1)], dtype=bool)


def attended_streaming(t: int, n_sink: int, n_local: int) -> np.ndarray:
    """Lambda mask at token granularity (Z11): the first n_sink tokens and
    the n_local most recent ones (t - p < n_local)."""
    p = np.arange(t + 1)
    return (p < n_sink) | ((t - p) < n_local)


# ---------------------------------------------------------------------------
# O8: decode attention output = dense masked softmax over the attended keys
# ---------------------------------------------------------------------------

def masked_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                     mask: np.ndarray, scale: float) -> np.ndarray:
    """o = sum_p softmax_p(scale * q.k_p) v_p over the p with mask[p].
    q: [D]; keys, values: [L][D]; mask: [L] bool (at least one True)."""
    idx = np.nonzero(mask)[0]
    logits = scale * (keys[idx] @ q)
    m = np.max(logits)
    w = np.exp(logits - m)
    return (w @ values[idx]) / np.sum(w)


# ---------------------------------------------------------------------------
# O6: the decode step sequence with reusable page selection
#     ([LS-X] Reusable Page Selection)
# ---------------------------------------------------------------------------

@dataclass
class DecodeSpec:
    num_q_heads: int
    num_kv_heads: int
    head_kind: Sequence[int]        # per KV head: 0 retrieval, 1 streaming
    logical_page: int               # N_L
    page_size: int                  # N_P
    token_budget: int               # K = token_budget / N_P pages
    reuse_interval: int             # R
    sink_tokens: int
    local_tokens: int
    scale: Optional[float] = None   # softmax scale; None -> 1/sqrt(D)
    aggregation: str = SUM          # how a GQA group's per-head page scores combine


def decode_step(spec: DecodeSpec, q: np.ndarray, keys: Sequence[np.ndarray],
                values: Sequence[np.ndarray], selected: Optional[np.ndarray],
                reselect: bool, key_codes: Optional[Sequence[np.ndarray]] = None):
    """One decode step of one sequence.

    q: [H_q][D] float64 query of the token at t = L - 1.
    keys/values: per KV head, [L][D] float64 of every cached token including t
      (the step's K/V has already been appended, Z14).
    selected: [H_kv][K] the selection kept from the previous step (or None).
    reselect: True at steps i with i % R == 0 (Z9).
    Returns (o [H_q][D], selected [H_kv][K]).  Streaming heads' rows of the
    selection are left as they were (Z16).
    """
    H_q, D = q.shape
    H_kv = spec.num_kv_heads
    G = H_q // H_kv
    g = spec.page_size // spec.logical_page
    K = spec.token_budget // spec.page_size
    scale = spec.scale if spec.scale else 1.0 / np.sqrt(D)
    L = keys[0].shape[0]
    t = L - 1
    sel = np.full((H_kv, K), -1, dtype=np.int32) if selected is None else selected.copy()
    out = np.zeros((H_q, D))
    for kv in range(H_kv):
        group = q[kv * G:(kv + 1) * G]          # kappa(h) = h // G  (Z3)
        if spec.head_kind[kv] == RETRIEVAL:
            if reselect:
                kmin, kmax = page_stats(keys[kv], spec.logical_page)
                sel[kv] = select_pages(group, kmin, kmax, g, K, spec.aggregation)
            mask = attended_retrieval(t, sel[kv], spec.page_size)
        else:
            mask = attended_streaming(t, spec.sink_tokens, spec.local_tokens)
        for h in range(G):
            out[kv * G + h] = masked_attention(group[h], keys[kv], values[kv], mask, scale)
    return out, sel


# ---------------------------------------------------------------------------
# O9: block-sparse prefill   ([LS-X] mermaid figure: streaming heads use sink +
#     local blocks, retrieval heads a static pattern in prefill)
# ---------------------------------------------------------------------------

def tile_visible(a: int, c: int, kind: int, sink_blocks: int, local_blocks: int) -> bool:
    """Is key tile c visible from query tile a?  Causal tiles c <= a; a
    streaming head keeps the first sink_blocks tiles and the local_blocks most
    recent tiles counting the diagonal one (reading Z12)."""
    if c > a:
        return False
    if kind == RETRIEVAL:
        return True
    return c < sink_blocks or (a - c) < local_blocks


def prefill_mask(T: int, block: int, kind: int, sink_blocks: int, local_blocks: int) -> np.ndarray:
    """Token-level visibility [T][T]: p <= t and the tile (t//B, p//B) visible."""
    n = -(-T // block)
    tiles = np.array([[tile_visible(a, c, kind, sink_blocks, local_blocks)
                       for c in range(n)] for a in range(n)], dtype=bool)
    t = np.arange(T)
    vis = tiles[t[:, None] // block, t[None, :] // block]
    return vis & (t[None, :] <= t[:, None])


def prefill_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, kind: int,
                      block: int, sink_blocks: int, local_blocks: int,
                      scale: float, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Masked softmax attention of one query head over one KV head.

    q: [T][D]; keys, values: [T][D].  Computes the rows listed in `rows`
    (all rows if None), one query tile at a time over that tile's visible key
    tiles.  Returns [len(rows)][D].
    """
    T, D = q.shape
    rows = range(T) if rows is None else rows
    out = np.empty((len(rows), D))
    n = -(-T // block)
    for r_i, t in enumerate(rows):
        a = t // block
        cols = [c for c in range(n) if tile_visible(a, c, kind, sink_blocks, local_blocks)]
        idx = np.concatenate([np.arange(c * block, min((c + 1) * block, T)) for c in cols])
        idx = idx[idx <= t]
        logits = scale * (keys[idx] @ q[t])
        m = np.max(logits)
        w = np.exp(logits - m)
        out[r_i] = (w @ values[idx]) / np.sum(w)
    return out


def block_mask_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, tile_mask: np.ndarray,
                         block: int, scale: float, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Softmax attention of one query head under an arbitrary static tile
    mask ([LS-X] 統一ブロックスパースアテンション: the kernel visits the
    non-empty tiles of a block-sparse pattern; reading Z26: any pattern of
    tiles at or below the diagonal, with the token-level causal rule p <= t
    kept inside every tile).

    tile_mask: [n][n] bool, n = ceil(T / block); query t sees key p iff
    tile_mask[t // block][p // block] and p <= t.  A query that sees no key
    gets the zero vector (reading Z27).  Returns [len(rows)][D].
    """
    T, D = q.shape
    rows = range(T) if rows is None else rows
    out = np.zeros((len(rows), D))
    for r_i, t in enumerate(rows):
        a = t // block
        idx = np.array([p for p in range(t + 1) if tile_mask[a, p // block]], dtype=np.int64)
        if idx.size == 0:
            continue
        logits = scale * (keys[idx] @ q[t])
        m = np.max(logits)
        w = np.exp(logits - m)
        out[r_i] = (w @ values[idx]) / np.sum(w)
    return out


def kind_tile_mask(n_blocks: int, kind: int, sink_blocks: int, local_blocks: int) -> np.ndarray:
    """The tile mask [n][n] of a head kind (the figure's causal and Lambda patterns)."""
    return np.array([[tile_visible(a, c, kind, sink_blocks, local_blocks) for c in range(n_blocks)]
                     for a in range(n_blocks)], dtype=bool)


# ---------------------------------------------------------------------------
# O10: block accounting and the theoretical speed-up 1/(1-r)
#      ([LS-X] 統一ブロックスパースアテンション)
# ---------------------------------------------------------------------------

def block_counts(n_blocks: int, kind: int, sink_blocks: int, local_blocks: int):
    """(non-empty tiles, causal tiles) of one head's n x n tile grid."""
    nnz = sum(1 for a in range(n_blocks) for c in range(a + 1)
              if tile_visible(a, c, kind, sink_blocks, local_blocks))
    return nnz, n_blocks * (n_blocks + 1) // 2


def sparsity_and_speedup(nnz: int, dense: int):
    """Block sparsity r = 1 - nnz/dense and the speed-up 1/(1-r), as exact
    fractions."""
    r = 1 - Fraction(nnz, dense)
    return r, 1 / (1 - r)


def mask_sparsity(tile_mask: np.ndarray):
    """r and 1/(1-r) of an explicit lower-triangular tile mask [n][n]."""
    n = tile_mask.shape[0]
    nnz = int(sum(bool(tile_mask[a, c]) for a in range(n) for c in range(a + 1)))
    return sparsity_and_speedup(nnz, n * (n + 1) // 2)
