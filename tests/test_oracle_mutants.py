"""Planted mistakes in the oracle, on the CPU: each mutant below is a
plausible slip (a dropped term, a wrong sign or index, min for max, an
off-by-one window) and must make at least one of the pins fail.  This shows
the pins can catch what they are meant to catch."""
from fractions import Fraction

import numpy as np
import pytest

import oracle.lsa_oracle as O
import tests.test_oracle_pins as P


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, IndexError, ValueError):
        return True
    return False


# --- scores ----------------------------------------------------------------

def score_min_not_max(q, kmin, kmax):
    q = np.asarray(q, float)
    return sum(np.sum(np.minimum(q[h] * kmax, q[h] * kmin), axis=1) for h in range(q.shape[0]))


def score_drops_last_head(q, kmin, kmax):
    q = np.asarray(q, float)
    return sum((np.sum(np.maximum(q[h] * kmax, q[h] * kmin), axis=1) for h in range(q.shape[0] - 1)),
               np.zeros(kmin.shape[0]))


def score_kmax_only(q, kmin, kmax):
    q = np.asarray(q, float)
    return sum(kmax @ q[h] for h in range(q.shape[0]))


def score_max_over_heads(q, kmin, kmax):
    q = np.asarray(q, float)
    return np.max([np.sum(np.maximum(q[h] * kmax, q[h] * kmin), axis=1) for h in range(q.shape[0])], axis=0)


def score_mean_center(q, kmin, kmax):
    q = np.asarray(q, float)
    return sum(((kmin + kmax) / 2) @ q[h] for h in range(q.shape[0]))


@pytest.mark.parametrize("mutant", [score_min_not_max, score_drops_last_head, score_kmax_only,
                                    score_max_over_heads, score_mean_center])
def test_score_mutants_caught(mutant):
    caught = (_fails(P.pin_score_is_box_support, mutant)
              or _fails(P.pin_score_upper_bound, mutant, O.page_stats)
              or _fails(P.pin_score_special_cases, mutant))
    assert caught


def _agg(per_head_fn):
    """A logical_scores stand-in whose "max" path is per_head_fn (the "sum"
    path is the oracle's)."""
    def f(q, kmin, kmax, aggregation="sum"):
        if aggregation == "sum":
            return O.logical_scores(q, kmin, kmax)
        q = np.asarray(q, float)
        per = np.array([np.sum(np.maximum(q[h] * kmax, q[h] * kmin), axis=1) for h in range(q.shape[0])])
        return per_head_fn(per)
    return f


@pytest.mark.parametrize("mutant", [
    _agg(lambda per: per.sum(axis=0)),            # sums although max was asked for
    _agg(lambda per: per.mean(axis=0)),           # mean of the heads
    _agg(lambda per: per[0]),                     # first head only
    _agg(lambda per: per.min(axis=0)),            # min for max
])
def test_score_max_aggregation_mutants_caught(mutant):
    assert _fails(P.pin_score_max_aggregation, mutant, O.page_stats)


# --- stats -----------------------------------------------------------------

def stats_shifted(keys, n_l):
    L, D = keys.shape
    n = -(-L // n_l)
    kmin = np.array([keys[j * n_l + 1: min((j + 1) * n_l + 1, L)].min(0) if j * n_l + 1 < L
                     else keys[-1] for j in range(n)])
    kmax = np.array([keys[j * n_l + 1: min((j + 1) * n_l + 1, L)].max(0) if j * n_l + 1 < L
                     else keys[-1] for j in range(n)])
    return kmin, kmax


def stats_drop_tail(keys, n_l):
    L, D = keys.shape
    n = L // n_l
    return (np.array([keys[j * n_l:(j + 1) * n_l].min(0) for j in range(n)]),
            np.array([keys[j * n_l:(j + 1) * n_l].max(0) for j in range(n)]))


@pytest.mark.parametrize("mutant", [stats_shifted, stats_drop_tail])
def test_stats_mutants_caught(mutant):
    assert _fails(P.pin_stats_brute_force, mutant) or _fails(P.pin_score_upper_bound, O.logical_scores, mutant)


# --- physical max ----------------------------------------------------------

def phys_mean(S, g):
    n = len(S)
    return np.array([np.mean(S[m * g:min((m + 1) * g, n)]) for m in range(-(-n // g))])


def phys_off_by_one(S, g):
    n = len(S)
    return np.array([np.max(S[m * g:min((m + 1) * g + 1, n)]) for m in range(-(-n // g))])


def phys_drop_tail(S, g):
    n = len(S)
    return np.array([np.max(S[m * g:(m + 1) * g]) for m in range(n // g)])


@pytest.mark.parametrize("mutant", [phys_mean, phys_off_by_one, phys_drop_tail])
def test_physical_mutants_caught(mutant):
    assert _fails(P.pin_physical_is_max, mutant)


# --- top-K -----------------------------------------------------------------

def topk_ties_high(P_, k):
    n = len(P_)
    order = sorted(range(n), key=lambda m: (-P_[m], -m))
    out = np.full(k, -1, np.int32)
    ch = sorted(order[:k])
    out[:len(ch)] = ch
    return out


def topk_descending_output(P_, k):
    n = len(P_)
    order = sorted(range(n), key=lambda m: (-P_[m], m))[:k]
    out = np.full(k, -1, np.int32)
    out[:len(order)] = order
    return out


def topk_smallest(P_, k):
    return O.topk_pages(-np.asarray(P_), k)


def topk_k_minus_one(P_, k):
    out = O.topk_pages(P_, k - 1)
    return np.concatenate([out, [-1]]).astype(np.int32)


@pytest.mark.parametrize("mutant", [topk_ties_high, topk_descending_output, topk_smallest, topk_k_minus_one])
def test_topk_mutants_caught(mutant):
    assert _fails(P.pin_topk, mutant)


# --- attention and masks ---------------------------------------------------

def attn_no_scale(q, k, v, mask, scale):
    return O.masked_attention(q, k, v, mask, 1.0)


def attn_ignores_mask(q, k, v, mask, scale):
    return O.masked_attention(q, k, v, np.ones_like(mask), scale)


def attn_keys_as_values(q, k, v, mask, scale):
    idx = np.nonzero(mask)[0]
    lg = scale * (k[idx] @ q)
    w = np.exp(lg - lg.max())
    return (w @ k[idx]) / w.sum()


@pytest.mark.parametrize("mutant", [attn_no_scale, attn_ignores_mask, attn_keys_as_values])
def test_attention_mutants_caught(mutant):
    assert _fails(P.pin_masked_attention, mutant)


def stream_off_by_one(t, ns, nl):
    p = np.arange(t + 1)
    return (p < ns) | ((t - p) <= nl)


def stream_no_sink(t, ns, nl):
    p = np.arange(t + 1)
    return (t - p) < nl


def retrieval_without_current(t, sel, n_p):
    pages = set(int(m) for m in sel if m >= 0)
    return np.array([(p // n_p) in pages for p in range(t + 1)], dtype=bool)


def test_mask_mutants_caught():
    assert _fails(P.pin_streaming_mask, stream_off_by_one)
    assert _fails(P.pin_streaming_mask, stream_no_sink)
    assert _fails(P.pin_retrieval_set, retrieval_without_current)


def prefill_local_off_by_one(q, k, v, kind, B, sb, lb, sc, rows=None):
    return O.prefill_attention(q, k, v, kind, B, sb, lb + 1, sc, rows)


def prefill_no_diag_causal(q, k, v, kind, B, sb, lb, sc, rows=None):
    T, D = q.shape
    out = np.empty((T, D))
    n = -(-T // B)
    for t in range(T):
        a = t // B
        cols = [c for c in range(n) if O.tile_visible(a, c, kind, sb, lb)]
        idx = np.concatenate([np.arange(c * B, min((c + 1) * B, T)) for c in cols])
        lg = sc * (k[idx] @ q[t])
        w = np.exp(lg - lg.max())
        out[t] = (w @ v[idx]) / w.sum()
    return out


@pytest.mark.parametrize("mutant", [prefill_local_off_by_one, prefill_no_diag_causal])
def test_prefill_mutants_caught(mutant):
    assert _fails(P.pin_prefill, mutant)


def mask_transposed(q, k, v, m, B, sc, rows=None):
    return O.block_mask_attention(q, k, v, m.T, B, sc, rows)


def mask_no_token_causal(q, k, v, m, B, sc, rows=None):
    T, D = q.shape
    rows = range(T) if rows is None else rows
    out = np.zeros((len(rows), D))
    for i, t in enumerate(rows):
        idx = np.array([p for p in range(T) if m[t // B, p // B]], dtype=np.int64)
        if idx.size:
            lg = sc * (k[idx] @ q[t])
            w = np.exp(lg - lg.max())
            out[i] = (w @ v[idx]) / w.sum()
    return out


def mask_tile_index_shifted(q, k, v, m, B, sc, rows=None):
    T, D = q.shape
    rows = range(T) if rows is None else rows
    out = np.zeros((len(rows), D))
    for i, t in enumerate(rows):
        idx = np.array([p for p in range(t + 1) if m[t // B, (p + 1) // B if (p + 1) // B < m.shape[1] else p // B]],
                       dtype=np.int64)
        if idx.size:
            lg = sc * (k[idx] @ q[t])
            w = np.exp(lg - lg.max())
            out[i] = (w @ v[idx]) / w.sum()
    return out


def mask_empty_row_uniform(q, k, v, m, B, sc, rows=None):
    out = O.block_mask_attention(q, k, v, m, B, sc, rows)
    T = q.shape[0]
    rows = list(range(T)) if rows is None else list(rows)
    for i, t in enumerate(rows):
        if not m[t // B].any():
            out[i] = v[: t + 1].mean(axis=0)
    return out


@pytest.mark.parametrize("mutant", [mask_transposed, mask_no_token_causal, mask_tile_index_shifted,
                                    mask_empty_row_uniform])
def test_block_mask_mutants_caught(mutant):
    assert _fails(P.pin_block_mask, mutant)


def counts_square(n, kind, sb, lb):
    nnz, _ = O.block_counts(n, kind, sb, lb)
    return nnz, n * n


def speedup_inverted(nnz, dense):
    r = Fraction(nnz, dense)
    return r, 1 / (1 - r)


def test_accounting_mutants_caught():
    assert _fails(P.pin_block_accounting, counts_square, O.sparsity_and_speedup)
    assert _fails(P.pin_block_accounting, O.block_counts, speedup_inverted)


# --- KV4 dequantisation ----------------------------------------------------

def dequant_scale_then_zero(codes, s, z):
    return np.asarray(codes, np.float64) * s - z


def dequant_plus_zero(codes, s, z):
    return (np.asarray(codes, np.float64) + z) * s


def dequant_divides_by_scale(codes, s, z):
    return (np.asarray(codes, np.float64) - z) / s


@pytest.mark.parametrize("mutant", [dequant_scale_then_zero, dequant_plus_zero, dequant_divides_by_scale])
def test_dequant_mutants_caught(mutant):
    assert _fails(P.pin_dequant_int4, mutant)


# --- the decode step's reselect path -----------------------------------------

def decode_step_stats_before_current(spec, q, keys, values, selected, reselect, key_codes=None):
    """Builds the selection statistics from keys[:t], leaving out the current token."""
    orig = O.page_stats
    O.page_stats = lambda k, n_l: orig(k[:-1], n_l)
    try:
        return O.decode_step(spec, q, keys, values, selected, reselect)
    finally:
        O.page_stats = orig


def decode_step_always_reselects(spec, q, keys, values, selected, reselect, key_codes=None):
    return O.decode_step(spec, q, keys, values, selected, True)


def decode_step_drops_current_page(spec, q, keys, values, selected, reselect, key_codes=None):
    """Attends the selected pages only, not the page of the current token."""
    orig = O.attended_retrieval

    def no_current(t, sel, n_p):
        pages = set(int(m) for m in sel if m >= 0)
        return np.array([(p // n_p) in pages for p in range(t + 1)], dtype=bool)
    O.attended_retrieval = no_current
    try:
        return O.decode_step(spec, q, keys, values, selected, reselect)
    finally:
        O.attended_retrieval = orig


def decode_step_scores_first_head_only(spec, q, keys, values, selected, reselect, key_codes=None):
    orig = O.select_pages
    O.select_pages = lambda qg, kmin, kmax, g, k, agg=O.SUM: orig(qg[:1], kmin, kmax, g, k, agg)
    try:
        return O.decode_step(spec, q, keys, values, selected, reselect)
    finally:
        O.select_pages = orig


@pytest.mark.parametrize("mutant", [decode_step_stats_before_current, decode_step_always_reselects,
                                    decode_step_drops_current_page, decode_step_scores_first_head_only])
def test_decode_step_mutants_caught(mutant):
    assert _fails(P.pin_decode_step_partial_budget, mutant)
