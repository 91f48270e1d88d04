// Host side of the C ABI declared in include/lsa.h: argument validation,
// workspace sizing, work decomposition and kernel dispatch.  Nothing here
// allocates device memory or synchronises the host.
#include <algorithm>
#include <cmath>
#include <utility>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "lsa_internal.h"

namespace lsa {
namespace {

thread_local std::string g_last_error;

lsa_status fail(lsa_status code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

lsa_status ok() {
    g_last_error.clear();
    return LSA_OK;
}

lsa_status from_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(LSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

lsa_status check_kv(const lsa_kv *kv) {
    if (!kv) return fail(LSA_ERR_INVALID_ARG, "kv descriptor is NULL");
    if (kv->kv_dtype != LSA_F32 && kv->kv_dtype != LSA_BF16 && kv->kv_dtype != LSA_INT4)
        return fail(LSA_ERR_INVALID_ARG, "kv_dtype %d is not LSA_F32, LSA_BF16 or LSA_INT4", kv->kv_dtype);
    if (kv->reserved != 0) return fail(LSA_ERR_INVALID_ARG, "kv->reserved must be 0");
    if (kv->num_kv_heads < 1 || kv->num_kv_heads > kMaxKvHeads)
        return fail(LSA_ERR_UNSUPPORTED, "num_kv_heads %d outside [1, %d]", kv->num_kv_heads, kMaxKvHeads);
    if (kv->head_dim != 64 && kv->head_dim != 128)
        return fail(LSA_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", kv->head_dim);
    if (kv->logical_page != 8 && kv->logical_page != 16 && kv->logical_page != 32 && kv->logical_page != 64)
        return fail(LSA_ERR_UNSUPPORTED, "logical_page %d is not 8, 16, 32 or 64", kv->logical_page);
    if (kv->page_size < kv->logical_page || kv->page_size % kv->logical_page != 0)
        return fail(LSA_ERR_INVALID_ARG, "page_size %d is not a multiple of logical_page %d", kv->page_size,
                    kv->logical_page);
    if (kv->page_size < 16 || kv->page_size > 256 || !is_pow2(kv->page_size))
        return fail(LSA_ERR_UNSUPPORTED, "page_size %d: need 16, 32, 64, 128 or 256", kv->page_size);
    if (kv->num_pages < 1) return fail(LSA_ERR_INVALID_ARG, "num_pages must be >= 1");
    if (!kv->k || !kv->v) return fail(LSA_ERR_INVALID_ARG, "kv->k and kv->v must be non-NULL");
    if (kv->kv_dtype == LSA_INT4) {
        if (!kv->k_sz || !kv->v_sz) return fail(LSA_ERR_INVALID_ARG, "int4 pool needs k_sz and v_sz");
    } else if (kv->k_sz || kv->v_sz) {
        return fail(LSA_ERR_INVALID_ARG, "k_sz / v_sz are for int4 pools only");
    }
    return LSA_OK;
}

lsa_status check_seqs(const lsa_seqs *sq) {
    if (!sq) return fail(LSA_ERR_INVALID_ARG, "seqs descriptor is NULL");
    if (sq->batch < 0) return fail(LSA_ERR_INVALID_ARG, "batch %d < 0", sq->batch);
    if (sq->max_pages < 1 || sq->max_pages > 65535)
        return fail(LSA_ERR_UNSUPPORTED, "max_pages %d outside [1, 65535]", sq->max_pages);
    if (sq->batch > 0 && (!sq->page_table || !sq->seq_lens))
        return fail(LSA_ERR_INVALID_ARG, "page_table and seq_lens must be non-NULL");
    return LSA_OK;
}

lsa_status check_heads(const lsa_heads *hd, const lsa_kv *kv, bool need) {
    if (!hd) return need ? fail(LSA_ERR_INVALID_ARG, "heads descriptor is NULL") : LSA_OK;
    if (!hd->head_kind) return fail(LSA_ERR_INVALID_ARG, "heads->head_kind is NULL");
    if (hd->num_q_heads < 1 || hd->num_q_heads % kv->num_kv_heads != 0)
        return fail(LSA_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                    hd->num_q_heads, kv->num_kv_heads);
    if (hd->num_q_heads / kv->num_kv_heads > 16)
        return fail(LSA_ERR_UNSUPPORTED, "GQA group size %d > 16", hd->num_q_heads / kv->num_kv_heads);
    for (int i = 0; i < kv->num_kv_heads; ++i)
        if (hd->head_kind[i] > 1) return fail(LSA_ERR_INVALID_ARG, "head_kind[%d] = %d is not 0 or 1", i, hd->head_kind[i]);
    if (hd->sink_tokens < 0 || hd->local_tokens < 1)
        return fail(LSA_ERR_INVALID_ARG, "need sink_tokens >= 0 and local_tokens >= 1");
    if (hd->sink_blocks < 0 || hd->local_blocks < 1)
        return fail(LSA_ERR_INVALID_ARG, "need sink_blocks >= 0 and local_blocks >= 1");
    if (hd->score_aggregation != LSA_AGG_SUM && hd->score_aggregation != LSA_AGG_MAX)
        return fail(LSA_ERR_INVALID_ARG, "score_aggregation %d is not LSA_AGG_SUM or LSA_AGG_MAX",
                    hd->score_aggregation);
    return LSA_OK;
}

int count_kind(const lsa_heads *hd, int h_kv, int kind) {
    int n = 0;
    for (int i = 0; i < h_kv; ++i) n += hd->head_kind[i] == kind;
    return n;
}

// The head map of a layer: the streaming heads as a bit mask, and the head
// slots of the pool: every KV head, or only the retrieval heads (in KV-head
// order) when the streaming heads live in a stream cache.
void pool_heads_of(const lsa_kv *kv, const lsa_heads *hd, HeadMap &hm, int *n_str = nullptr) {
    hm.str_mask = 0;
    int r = 0, st = 0;
    for (int i = 0; i < kv->num_kv_heads; ++i) {
        const bool ret = !hd || hd->head_kind[i] == LSA_RETRIEVAL_HEAD;
        if (!ret) hm.str_mask |= 1ull << i;
        r += ret;
        st += !ret;
    }
    hm.pool_heads = kv->stream_cache ? r : kv->num_kv_heads;
    hm.by_rank = kv->stream_cache ? 1 : 0;
    if (n_str) *n_str = st;
}

lsa_status check_stream_cache(const lsa_stream_cache *sc, const lsa_kv *kv, const lsa_heads *hd) {
    if (!hd) return fail(LSA_ERR_INVALID_ARG, "a pool with a stream cache needs the head classification");
    if (sc->sink_pages < 0 || sc->ring_pages < 1)
        return fail(LSA_ERR_INVALID_ARG, "stream cache: sink_pages %d, ring_pages %d", sc->sink_pages, sc->ring_pages);
    const int NP = kv->page_size;
    const int need_sink = (hd->sink_tokens + NP - 1) / NP, need_ring = (hd->local_tokens + NP - 1) / NP + 1;
    if (sc->sink_pages < need_sink || sc->ring_pages < need_ring)
        return fail(LSA_ERR_INVALID_ARG,
                    "stream cache of %d sink + %d ring pages cannot hold %d sink + %d local tokens (need %d + %d)",
                    sc->sink_pages, sc->ring_pages, hd->sink_tokens, hd->local_tokens, need_sink, need_ring);
    if (!sc->k || !sc->v) return fail(LSA_ERR_INVALID_ARG, "stream cache k and v must be non-NULL");
    if ((kv->kv_dtype == LSA_INT4) != (sc->k_sz != nullptr && sc->v_sz != nullptr))
        return fail(LSA_ERR_INVALID_ARG, "stream cache k_sz / v_sz are needed for int4 pools and only for them");
    return LSA_OK;
}

// Validation of a pool descriptor together with the head classification.
lsa_status check_pool(const lsa_kv *kv, const lsa_heads *hd) {
    if (kv->stream_cache) return check_stream_cache(kv->stream_cache, kv, hd);
    return LSA_OK;
}

struct DecodeGeom {
    int K, chunk_pages, chunks_ret, chunks_str, chunks_max, rec_floats;
};

// arrival counters at the start of the decode workspace: one int32 per (sequence, KV head)
size_t decode_counter_bytes(int batch, int num_kv_heads) { return align_up((size_t)batch * num_kv_heads * 4); }

// Chunks of a (sequence, KV head): its attended pages, at most the kernel's
// chunk size per workgroup.  A launch that fits the chip's workgroup slots in
// one round takes smaller chunks while it still fits, its last workgroups
// still merge a head's records in one batch, and at least three of a
// workgroup's four wavefronts still have pages: workgroups reach the CUs one
// per CU per round, so the 384 workgroups of 8 pages of a B = 8, 64K-token
// layer (8 KV heads, half of them streaming, a 4096-token budget) put 16 pages on
// half of the CUs, whose second workgroups then finish their streams about
// 5 us after the others (448 workgroups of 6 pages: at most 12 pages per CU;
// 21.5 us per launch against 23.1).  Chunks that leave two wavefronts idle
// were slower (256-token pages at two per chunk: 24.1 against 22.3 us).
DecodeGeom decode_geometry(const lsa_kv *kv, const lsa_heads *hd, int token_budget, int batch) {
    DecodeGeom g;
    g.K = token_budget / kv->page_size;
    const int per_chunk = decode_chunk_pages(kv->kv_dtype, kv->page_size);
    const int NP = kv->page_size;
    const int ret_pages = g.K + 1;
    const int str_pages = (hd->sink_tokens + NP - 1) / NP + (hd->local_tokens - 1) / NP + 2;
    const int n_ret = count_kind(hd, kv->num_kv_heads, LSA_RETRIEVAL_HEAD);
    const int n_str = kv->num_kv_heads - n_ret;
    auto cdiv = [](int x, int y) { return (x + y - 1) / y; };
    auto wgs = [&](int c) { return (long long)batch * (n_ret * cdiv(ret_pages, c) + n_str * cdiv(str_pages, c)); };
    auto most = [&](int c) { return std::max(n_ret ? cdiv(ret_pages, c) : 0, n_str ? cdiv(str_pages, c) : 0); };
    int cp = per_chunk;
    if (kv->kv_dtype != LSA_F32) {
        const int ppw = decode_pages_per_wave(kv->kv_dtype, NP);
        const long long slots = (long long)decode_waves_per_simd(kv->kv_dtype, NP) * kComputeUnits;
        if (wgs(cp) <= slots)
            while (cp - 1 > 2 * ppw && wgs(cp - 1) <= slots && most(cp - 1) <= kDecodeMergeBatch) --cp;
    }
    g.chunk_pages = cp;
    g.chunks_ret = cdiv(ret_pages, cp);
    g.chunks_str = cdiv(str_pages, cp);
    g.chunks_max = std::max(g.chunks_ret, g.chunks_str);
    g.rec_floats = 32 + (hd->num_q_heads / kv->num_kv_heads) * kv->head_dim;
    return g;
}

// Validation and the shared fields of a prefill launch (both mask kinds).
lsa_status prefill_setup(PrefillArgs &p, const void *q, int32_t q_dtype, const lsa_kv *kv, const int32_t *page_table,
                         int32_t seq_len, int32_t num_q_heads, int32_t block, float softmax_scale, void *out,
                         int64_t *tile_counter, bool &empty) {
    if (block != 64) return fail(LSA_ERR_UNSUPPORTED, "block %d: only 64-token tiles are built", block);
    if (kv->stream_cache)
        return fail(LSA_ERR_UNSUPPORTED, "prefill reads every head from the pool: pass a pool without a stream cache");
    if (kv->page_size % 64 != 0)
        return fail(LSA_ERR_UNSUPPORTED, "prefill needs page_size a multiple of 64 (got %d)", kv->page_size);
    const bool pair_ok = (q_dtype == LSA_F32 && kv->kv_dtype == LSA_F32) ||
                         (q_dtype == LSA_BF16 && kv->kv_dtype == LSA_BF16);
    if (!pair_ok)
        return fail(LSA_ERR_UNSUPPORTED, "(q_dtype %d, kv_dtype %d) is not a supported prefill pair", q_dtype,
                    kv->kv_dtype);
    if (q_dtype == LSA_F32 && kv->head_dim != 64)
        return fail(LSA_ERR_UNSUPPORTED, "f32 prefill is built for head_dim 64 only");
    if (seq_len < 0) return fail(LSA_ERR_INVALID_ARG, "seq_len %d < 0", seq_len);
    if (!q || !out || (seq_len > 0 && !page_table))
        return fail(LSA_ERR_INVALID_ARG, "q, out and page_table must be non-NULL");
    if (!(softmax_scale >= 0.f) || std::isinf(softmax_scale))
        return fail(LSA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    empty = seq_len == 0;
    p.q = q;
    p.out = out;
    p.k = kv->k;
    p.v = kv->v;
    p.page_table = page_table;
    p.tile_counter = reinterpret_cast<unsigned long long *>(tile_counter);
    p.seq_len = seq_len;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = kv->num_kv_heads;
    p.group = num_q_heads / kv->num_kv_heads;
    p.head_dim = kv->head_dim;
    p.page_size = kv->page_size;
    p.n_qblocks = (seq_len + 63) / 64;
    p.head_groups = (p.group + 3) / 4;
    p.q_tiles = 1;
    p.n_qgroups = p.n_qblocks;
    p.n_ret = 0;
    p.n_str = 0;
    const long long items = (long long)kv->num_kv_heads * p.n_qblocks * p.head_groups;
    if (items > (long long)INT32_MAX) return fail(LSA_ERR_UNSUPPORTED, "prefill launch too large");
    p.n_items = (int32_t)items;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / std::sqrt((float)kv->head_dim);
    p.scale_log2 = scale * 1.4426950408889634f;
    return LSA_OK;
}

// ---------------------------------------------------------------------------
// Static scratch of lsa_sparse_decode_attn_noalloc: the decode workspace
// (arrival counters, then the split-KV partial records) in a file-scope device
// array, for callers that cannot allocate.  Each GPU the library runs on holds
// its own copy until the process ends; every call on that GPU shares it.
// Host code addresses it only through the pointer hipGetSymbolAddress returns
// for the current device (the array's name is a host-side stand-in).
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The address of the current device's copy of the scratch array, looked up
// once per device (with that device current) and kept.
lsa_status static_scratch(void **out) {
    int dev = -1;
    if (hipError_t e = hipGetDevice(&dev)) return from_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(LSA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return from_hip(e, "hipGetSymbolAddress");
        if (!p) return fail(LSA_ERR_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LSA_OK;
}

__global__ void zero_i32_kernel(int32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// The newest token's rows that a decode step appends (all NULL: none).
struct NewToken {
    const void *k = nullptr, *v = nullptr;
    const uint16_t *k_sz = nullptr, *v_sz = nullptr;
};

lsa_status decode_attn_impl(const void *q, int32_t q_dtype, const lsa_kv *kv, const lsa_seqs *seqs,
                            const lsa_heads *heads, const int32_t *selected, int32_t token_budget,
                            float softmax_scale, void *out, void *stats, void *workspace, size_t workspace_bytes,
                            bool clear_counters, const NewToken &nt, hipStream_t stream, bool check_only = false);

lsa_status select_impl(const void *q, int32_t q_dtype, const lsa_kv *kv, const void *stats, const lsa_seqs *seqs,
                       const lsa_heads *heads, int32_t token_budget, int32_t decode_step, int32_t reuse_interval,
                       int32_t *selected, void *workspace, size_t workspace_bytes, const NewToken &nt,
                       hipStream_t stream, bool check_only = false);

lsa_status check_new_token(const lsa_kv *kv, const NewToken &nt) {
    if (!nt.k || !nt.v) return fail(LSA_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
    if ((kv->kv_dtype == LSA_INT4) != (nt.k_sz != nullptr && nt.v_sz != nullptr))
        return fail(LSA_ERR_INVALID_ARG, "k_new_sz / v_new_sz are needed for int4 pools and only for them");
    return LSA_OK;
}

}  // namespace
}  // namespace lsa

using namespace lsa;

extern "C" {

const char *lsa_last_error(void) { return g_last_error.c_str(); }

#ifndef LSA_SOURCE_SHA
#define LSA_SOURCE_SHA "unknown"
#endif
const char *lsa_version(void) { return "lsa 0.2.0 gfx950 src " LSA_SOURCE_SHA; }

lsa_status lsa_page_stats_bytes(const lsa_kv *kv, const lsa_heads *heads, size_t *bytes) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_heads(heads, kv, kv->stream_cache != nullptr)) return s;
    if (lsa_status s = check_pool(kv, heads)) return s;
    if (!bytes) return fail(LSA_ERR_INVALID_ARG, "bytes is NULL");
    HeadMap hm;
    pool_heads_of(kv, heads, hm);
    const size_t g = kv->page_size / kv->logical_page;
    const size_t per = kv->kv_dtype == LSA_INT4 ? (size_t)kv->head_dim
                                                 : 2 * (size_t)kv->head_dim * (kv->kv_dtype == LSA_F32 ? 4 : 2);
    *bytes = (size_t)kv->num_pages * hm.pool_heads * g * per;
    return ok();
}

lsa_status lsa_stream_cache_pages(const lsa_kv *kv, const lsa_heads *heads, int32_t *sink_pages,
                                  int32_t *ring_pages) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_heads(heads, kv, true)) return s;
    if (!sink_pages || !ring_pages) return fail(LSA_ERR_INVALID_ARG, "sink_pages and ring_pages must be non-NULL");
    const int NP = kv->page_size;
    *sink_pages = (heads->sink_tokens + NP - 1) / NP;
    *ring_pages = (heads->local_tokens + NP - 1) / NP + 1;
    return ok();
}

lsa_status lsa_stream_cache_fill(const lsa_kv *src, const lsa_seqs *seqs, const lsa_heads *heads,
                                 const lsa_stream_cache *cache, void *stream) {
    if (lsa_status s = check_kv(src)) return s;
    if (lsa_status s = check_seqs(seqs)) return s;
    if (lsa_status s = check_heads(heads, src, true)) return s;
    if (src->stream_cache) return fail(LSA_ERR_INVALID_ARG, "the source pool must hold every head");
    if (!cache) return fail(LSA_ERR_INVALID_ARG, "cache is NULL");
    if (lsa_status s = check_stream_cache(cache, src, heads)) return s;
    FillArgs a{};
    a.k = src->k;
    a.v = src->v;
    a.k_sz = src->k_sz;
    a.v_sz = src->v_sz;
    a.page_table = seqs->page_table;
    a.seq_lens = seqs->seq_lens;
    a.sc_k = cache->k;
    a.sc_v = cache->v;
    a.sc_k_sz = cache->k_sz;
    a.sc_v_sz = cache->v_sz;
    a.batch = seqs->batch;
    a.max_pages = seqs->max_pages;
    a.num_kv_heads = src->num_kv_heads;
    a.head_dim = src->head_dim;
    a.page_size = src->page_size;
    a.dtype = src->kv_dtype;
    a.sc_sink = cache->sink_pages;
    a.sc_ring = cache->ring_pages;
    a.n_str = 0;
    for (int i = 0; i < src->num_kv_heads; ++i)
        if (heads->head_kind[i] == LSA_STREAMING_HEAD) a.str_heads[a.n_str++] = (uint8_t)i;
    if ((long long)a.batch * a.n_str * (a.sc_sink + a.sc_ring) > (long long)INT32_MAX)
        return fail(LSA_ERR_UNSUPPORTED, "stream cache too large");
    return from_hip(launch_stream_fill(a, (hipStream_t)stream), "stream cache fill launch");
}

lsa_status lsa_append_kv(const lsa_kv *kv, const lsa_seqs *seqs, const lsa_heads *heads, const void *k_new,
                         const void *v_new, const uint16_t *k_new_sz, const uint16_t *v_new_sz, void *stats,
                         void *stream) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_seqs(seqs)) return s;
    if (lsa_status s = check_heads(heads, kv, true)) return s;
    if (lsa_status s = check_pool(kv, heads)) return s;
    if (lsa_status s = check_new_token(kv, NewToken{k_new, v_new, k_new_sz, v_new_sz})) return s;
    AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_new_sz = k_new_sz;
    a.v_new_sz = v_new_sz;
    a.k = const_cast<void *>(kv->k);
    a.v = const_cast<void *>(kv->v);
    a.k_sz = const_cast<uint16_t *>(kv->k_sz);
    a.v_sz = const_cast<uint16_t *>(kv->v_sz);
    a.stats = stats;
    a.page_table = seqs->page_table;
    a.seq_lens = seqs->seq_lens;
    a.batch = seqs->batch;
    a.max_pages = seqs->max_pages;
    a.num_kv_heads = kv->num_kv_heads;
    a.head_dim = kv->head_dim;
    a.page_size = kv->page_size;
    a.logical_page = kv->logical_page;
    a.dtype = kv->kv_dtype;
    pool_heads_of(kv, heads, a.hm, &a.n_str);
    if (const lsa_stream_cache *sc = kv->stream_cache) {
        a.sc_k = sc->k;
        a.sc_v = sc->v;
        a.sc_k_sz = sc->k_sz;
        a.sc_v_sz = sc->v_sz;
        a.sc_sink = sc->sink_pages;
        a.sc_ring = sc->ring_pages;
    }
    return from_hip(launch_append(a, (hipStream_t)stream), "append launch");
}

lsa_status lsa_build_page_stats(const lsa_kv *kv, const lsa_seqs *seqs, const lsa_heads *heads,
                                const int32_t *first_token, int32_t max_new_tokens, void *stats,
                                void *stream) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_seqs(seqs)) return s;
    if (lsa_status s = check_heads(heads, kv, kv->stream_cache != nullptr)) return s;
    if (lsa_status s = check_pool(kv, heads)) return s;
    if (!stats) return fail(LSA_ERR_INVALID_ARG, "stats is NULL");
    if (max_new_tokens < 0) return fail(LSA_ERR_INVALID_ARG, "max_new_tokens < 0");
    StatsArgs a{};
    pool_heads_of(kv, heads, a.hm);
    a.k = kv->k;
    a.k_sz = kv->k_sz;
    a.stats = stats;
    a.page_table = seqs->page_table;
    a.seq_lens = seqs->seq_lens;
    a.first_token = first_token;
    a.batch = seqs->batch;
    a.max_pages = seqs->max_pages;
    a.num_kv_heads = kv->num_kv_heads;
    a.head_dim = kv->head_dim;
    a.page_size = kv->page_size;
    a.logical_page = kv->logical_page;
    a.dtype = kv->kv_dtype;
    a.n_heads_sel = 0;
    for (int i = 0; i < kv->num_kv_heads; ++i)
        if (!heads || heads->head_kind[i] == LSA_RETRIEVAL_HEAD) a.heads_sel[a.n_heads_sel++] = (uint8_t)i;
    const long long full = (long long)seqs->max_pages * (kv->page_size / kv->logical_page);
    long long lp = full;
    if (first_token) {
        const long long span = max_new_tokens > 0 ? max_new_tokens : (long long)seqs->max_pages * kv->page_size;
        lp = std::min(full, (span + kv->logical_page - 1) / kv->logical_page + 1);
    }
    a.lp_per_seq = (int32_t)lp;
    if ((long long)a.batch * a.n_heads_sel * lp > (long long)INT32_MAX)
        return fail(LSA_ERR_UNSUPPORTED, "statistics launch too large");
    return from_hip(launch_stats(a, (hipStream_t)stream), "build_page_stats launch");
}

lsa_status lsa_select_pages_workspace(const lsa_kv *kv, const lsa_seqs *seqs, const lsa_heads *heads,
                                      size_t *bytes) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_seqs(seqs)) return s;
    if (lsa_status s = check_heads(heads, kv, true)) return s;
    if (!bytes) return fail(LSA_ERR_INVALID_ARG, "bytes is NULL");
    // arrival counters of the fused top-K, then the physical page scores
    *bytes = decode_counter_bytes(seqs->batch, kv->num_kv_heads) +
             align_up((size_t)seqs->batch * kv->num_kv_heads * seqs->max_pages * sizeof(double));
    return ok();
}

lsa_status lsa_select_pages(const void *q, int32_t q_dtype, const lsa_kv *kv, const void *stats,
                            const lsa_seqs *seqs, const lsa_heads *heads, int32_t token_budget,
                            int32_t decode_step, int32_t reuse_interval, int32_t *selected,
                            void *workspace, size_t workspace_bytes, void *stream) {
    return select_impl(q, q_dtype, kv, stats, seqs, heads, token_budget, decode_step, reuse_interval, selected,
                       workspace, workspace_bytes, NewToken{}, (hipStream_t)stream);
}

lsa_status lsa_decode_workspace(const lsa_kv *kv, const lsa_seqs *seqs, const lsa_heads *heads,
                                int32_t token_budget, size_t *bytes) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_seqs(seqs)) return s;
    if (lsa_status s = check_heads(heads, kv, true)) return s;
    if (!bytes) return fail(LSA_ERR_INVALID_ARG, "bytes is NULL");
    if (token_budget < kv->page_size || token_budget % kv->page_size != 0)
        return fail(LSA_ERR_INVALID_ARG, "token_budget %d is not a positive multiple of page_size %d", token_budget,
                    kv->page_size);
    const DecodeGeom g = decode_geometry(kv, heads, token_budget, seqs->batch);
    *bytes = decode_counter_bytes(seqs->batch, kv->num_kv_heads) +
             align_up((size_t)seqs->batch * kv->num_kv_heads * g.chunks_max * g.rec_floats * sizeof(float));
    return ok();
}

lsa_status lsa_sparse_decode_attn(const void *q, int32_t q_dtype, const lsa_kv *kv, const lsa_seqs *seqs,
                                  const lsa_heads *heads, const int32_t *selected, int32_t token_budget,
                                  float softmax_scale, void *out, void *stats, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return decode_attn_impl(q, q_dtype, kv, seqs, heads, selected, token_budget, softmax_scale, out, stats,
                            workspace, workspace_bytes, false, NewToken{}, (hipStream_t)stream);
}

lsa_status lsa_sparse_decode_attn_noalloc(const void *q, int32_t q_dtype, const lsa_kv *kv, const lsa_seqs *seqs,
                                          const lsa_heads *heads, const int32_t *selected, int32_t token_budget,
                                          float softmax_scale, void *out, void *stats, void *stream) {
    return decode_attn_impl(q, q_dtype, kv, seqs, heads, selected, token_budget, softmax_scale, out, stats,
                            nullptr, 0, true, NewToken{}, (hipStream_t)stream);
}


lsa_status lsa_decode_step_workspace(const lsa_kv *kv, const lsa_seqs *seqs, const lsa_heads *heads,
                                     int32_t token_budget, size_t *bytes) {
    size_t sel = 0, dec = 0;
    if (lsa_status s = lsa_select_pages_workspace(kv, seqs, heads, &sel)) return s;
    if (lsa_status s = lsa_decode_workspace(kv, seqs, heads, token_budget, &dec)) return s;
    *bytes = std::max(sel, dec);
    return ok();
}

lsa_status lsa_decode_step(const void *q, int32_t q_dtype, const lsa_kv *kv, const lsa_seqs *seqs,
                           const lsa_heads *heads, const void *k_new, const void *v_new, const uint16_t *k_new_sz,
                           const uint16_t *v_new_sz, void *stats, int32_t token_budget, int32_t decode_step,
                           int32_t reuse_interval, int32_t *selected, float softmax_scale, void *out,
                           void *workspace, size_t workspace_bytes, void *stream) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_seqs(seqs)) return s;
    if (lsa_status s = check_heads(heads, kv, true)) return s;
    const NewToken nt{k_new, v_new, k_new_sz, v_new_sz};
    if (lsa_status s = check_new_token(kv, nt)) return s;
    const bool any_ret = count_kind(heads, kv->num_kv_heads, LSA_RETRIEVAL_HEAD) > 0;
    if (any_ret && !stats) return fail(LSA_ERR_INVALID_ARG, "stats is NULL but retrieval heads exist");
    size_t need = 0;
    if (lsa_status s = lsa_decode_step_workspace(kv, seqs, heads, token_budget, &need)) return s;
    if (!workspace || workspace_bytes < need)
        return fail(LSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    const hipStream_t st = (hipStream_t)stream;
    // every argument of both launches is checked before the first one
    if (any_ret)
        if (lsa_status s = select_impl(q, q_dtype, kv, stats, seqs, heads, token_budget, decode_step, reuse_interval,
                                       selected, workspace, workspace_bytes, nt, st, true))
            return s;
    if (lsa_status s = decode_attn_impl(q, q_dtype, kv, seqs, heads, selected, token_budget, softmax_scale, out,
                                        stats, workspace, workspace_bytes, false, nt, st, true))
        return s;
    // both launches start from zero arrival counters and leave them zero, so
    // they share the workspace in stream order
    if (any_ret) {
        if (lsa_status s = select_impl(q, q_dtype, kv, stats, seqs, heads, token_budget, decode_step, reuse_interval,
                                       selected, workspace, workspace_bytes, nt, st))
            return s;
    }
    return decode_attn_impl(q, q_dtype, kv, seqs, heads, selected, token_budget, softmax_scale, out, stats,
                            workspace, workspace_bytes, false, nt, st);
}

}  // extern "C"

namespace lsa {
namespace {

lsa_status select_impl(const void *q, int32_t q_dtype, const lsa_kv *kv, const void *stats, const lsa_seqs *seqs,
                       const lsa_heads *heads, int32_t token_budget, int32_t decode_step, int32_t reuse_interval,
                       int32_t *selected, void *workspace, size_t workspace_bytes, const NewToken &nt,
                       hipStream_t stream, bool check_only) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_seqs(seqs)) return s;
    if (lsa_status s = check_heads(heads, kv, true)) return s;
    if (q_dtype != LSA_F32 && q_dtype != LSA_BF16)
        return fail(LSA_ERR_INVALID_ARG, "q_dtype %d is not LSA_F32 or LSA_BF16", q_dtype);
    if (token_budget < kv->page_size || token_budget % kv->page_size != 0)
        return fail(LSA_ERR_INVALID_ARG, "token_budget %d is not a positive multiple of page_size %d", token_budget,
                    kv->page_size);
    if (reuse_interval < 1) return fail(LSA_ERR_INVALID_ARG, "reuse_interval %d < 1", reuse_interval);
    if (decode_step < 0) return fail(LSA_ERR_INVALID_ARG, "decode_step %d < 0", decode_step);
    if (lsa_status s = check_pool(kv, heads)) return s;
    if (!q || !stats || !selected) return fail(LSA_ERR_INVALID_ARG, "q, stats and selected must be non-NULL");
    size_t need = 0;
    lsa_select_pages_workspace(kv, seqs, heads, &need);
    if (!workspace || workspace_bytes < need)
        return fail(LSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (seqs->max_pages > topk_max_pages())
        return fail(LSA_ERR_UNSUPPORTED, "max_pages %d: page selection handles at most %d pages per sequence",
                    seqs->max_pages, topk_max_pages());
    if (check_only) return ok();
    if (decode_step % reuse_interval != 0) return ok();     // reuse the previous selection
    const int n_ret = count_kind(heads, kv->num_kv_heads, LSA_RETRIEVAL_HEAD);
    if (n_ret == 0 || seqs->batch == 0) return ok();

    ScoreArgs sa{};
    pool_heads_of(kv, heads, sa.hm);
    sa.q = q;
    sa.stats = stats;
    sa.k = kv->k;
    sa.k_sz = kv->k_sz;
    sa.k_new = nt.k;
    sa.k_new_sz = nt.k_sz;
    sa.page_table = seqs->page_table;
    sa.seq_lens = seqs->seq_lens;
    sa.counters = static_cast<int32_t *>(workspace);
    sa.phys = reinterpret_cast<double *>(static_cast<char *>(workspace) +
                                         decode_counter_bytes(seqs->batch, kv->num_kv_heads));
    sa.selected = selected;
    sa.k_pages = token_budget / kv->page_size;
    sa.fused_pt = score_fused_pt(seqs->max_pages, heads->score_aggregation == LSA_AGG_MAX);
    sa.batch = seqs->batch;
    sa.max_pages = seqs->max_pages;
    sa.num_q_heads = heads->num_q_heads;
    sa.num_kv_heads = kv->num_kv_heads;
    sa.head_dim = kv->head_dim;
    sa.page_size = kv->page_size;
    sa.logical_page = kv->logical_page;
    sa.q_dtype = q_dtype;
    sa.kv_dtype = kv->kv_dtype;
    sa.aggregation = heads->score_aggregation;
    sa.n_ret = n_ret;
    sa.pages_per_block =
        sa.aggregation == LSA_AGG_MAX
            ? score_pages_per_block(kv->kv_dtype, kv->head_dim, kv->page_size, kv->logical_page, sa.fused_pt, true)
            : score_loop_pages_per_block(seqs->batch, sa.n_ret, seqs->max_pages, kv->page_size, kv->logical_page,
                                         kv->kv_dtype);
    sa.blocks_per_head = (seqs->max_pages + sa.pages_per_block - 1) / sa.pages_per_block;
    if (lsa_status s = from_hip(launch_score(sa, stream), "select_pages score launch")) return s;
    if (sa.fused_pt > 0) return ok();              // the score kernel's last workgroups have selected

    TopkArgs ta{};
    ta.phys = sa.phys;
    ta.seq_lens = seqs->seq_lens;
    ta.selected = selected;
    ta.batch = seqs->batch;
    ta.max_pages = seqs->max_pages;
    ta.num_kv_heads = kv->num_kv_heads;
    ta.page_size = kv->page_size;
    ta.k = token_budget / kv->page_size;
    ta.n_ret = sa.n_ret;
    ta.hm = sa.hm;
    return from_hip(launch_topk(ta, stream), "select_pages top-K launch");
}

lsa_status decode_attn_impl(const void *q, int32_t q_dtype, const lsa_kv *kv, const lsa_seqs *seqs,
                            const lsa_heads *heads, const int32_t *selected, int32_t token_budget,
                            float softmax_scale, void *out, void *stats, void *workspace, size_t workspace_bytes,
                            bool use_static, const NewToken &nt, hipStream_t stream, bool check_only) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_seqs(seqs)) return s;
    if (lsa_status s = check_heads(heads, kv, true)) return s;
    const bool pair_ok = (q_dtype == LSA_F32 && kv->kv_dtype == LSA_F32) ||
                         (q_dtype == LSA_BF16 && kv->kv_dtype == LSA_BF16) ||
                         (q_dtype == LSA_BF16 && kv->kv_dtype == LSA_INT4);
    if (!pair_ok)
        return fail(LSA_ERR_UNSUPPORTED, "(q_dtype %d, kv_dtype %d) is not a supported pair", q_dtype, kv->kv_dtype);
    if (lsa_status s = check_pool(kv, heads)) return s;
    if (!q || !out) return fail(LSA_ERR_INVALID_ARG, "q and out must be non-NULL");
    const int n_ret = count_kind(heads, kv->num_kv_heads, LSA_RETRIEVAL_HEAD);
    if (n_ret > 0 && !selected) return fail(LSA_ERR_INVALID_ARG, "selected is NULL but retrieval heads exist");
    if (!(softmax_scale >= 0.f) || std::isinf(softmax_scale))
        return fail(LSA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    size_t need = 0;
    if (lsa_status s = lsa_decode_workspace(kv, seqs, heads, token_budget, &need)) return s;
    if (use_static && need > kStaticScratchBytes)
        return fail(LSA_ERR_UNSUPPORTED,
                    "lsa_sparse_decode_attn_noalloc: this batch needs %zu bytes of scratch, above the %zu-byte "
                    "static scratch array; use lsa_sparse_decode_attn with a caller workspace",
                    need, kStaticScratchBytes);
    if (!use_static && (!workspace || workspace_bytes < need))
        return fail(LSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    const DecodeGeom g = decode_geometry(kv, heads, token_budget, seqs->batch);
    if (g.chunks_max > kMaxDecodeChunks)
        return fail(LSA_ERR_UNSUPPORTED, "token budget / Lambda window spans %d split-KV chunks (limit %d)",
                    g.chunks_max, kMaxDecodeChunks);
    if (check_only) return ok();
    if (seqs->batch == 0) return ok();
    if (use_static)                       // every argument is valid: now touch the device
        if (lsa_status s = static_scratch(&workspace)) return s;
    DecodeArgs a{};
    a.q = q;
    a.out = out;
    a.k = kv->k;
    a.v = kv->v;
    a.k_sz = kv->k_sz;
    a.v_sz = kv->v_sz;
    a.page_table = seqs->page_table;
    a.seq_lens = seqs->seq_lens;
    a.selected = selected;
    a.counters = static_cast<int32_t *>(workspace);
    a.part = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                       decode_counter_bytes(seqs->batch, kv->num_kv_heads));
    a.stats = stats;
    a.k_new = nt.k;
    a.v_new = nt.v;
    a.k_new_sz = nt.k_sz;
    a.v_new_sz = nt.v_sz;
    a.logical_page = kv->logical_page;
    a.batch = seqs->batch;
    a.max_pages = seqs->max_pages;
    a.num_q_heads = heads->num_q_heads;
    a.num_kv_heads = kv->num_kv_heads;
    a.group = heads->num_q_heads / kv->num_kv_heads;
    a.head_dim = kv->head_dim;
    a.page_size = kv->page_size;
    a.sel_k = g.K;
    a.sink = heads->sink_tokens;
    a.local = heads->local_tokens;
    a.chunk_pages = g.chunk_pages;
    a.chunks_ret = g.chunks_ret;
    a.chunks_str = g.chunks_str;
    a.chunks_max = g.chunks_max;
    a.chunks_per_seq = n_ret * g.chunks_ret + (kv->num_kv_heads - n_ret) * g.chunks_str;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / std::sqrt((float)kv->head_dim);
    a.scale_log2 = scale * 1.4426950408889634f;
    pool_heads_of(kv, heads, a.hm, &a.n_str);
    if (const lsa_stream_cache *sc = kv->stream_cache) {
        a.sc_k = sc->k;
        a.sc_v = sc->v;
        a.sc_k_sz = sc->k_sz;
        a.sc_v_sz = sc->v_sz;
        a.sc_sink = sc->sink_pages;
        a.sc_ring = sc->ring_pages;
    }
    if (use_static) {
        // the static scratch keeps whatever the previous call left: zero the
        // arrival counters with a fill kernel (no memset node in a captured graph)
        const int n = seqs->batch * kv->num_kv_heads;
        hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a.counters, n);
        if (lsa_status s = from_hip(hipGetLastError(), "decode counter clear launch")) return s;
    }
    return from_hip(launch_decode(a, q_dtype, kv->kv_dtype, stream), "decode launch");
}

}  // namespace
}  // namespace lsa

extern "C" {

lsa_status lsa_sparse_prefill_attn(const void *q, int32_t q_dtype, const lsa_kv *kv, const int32_t *page_table,
                                   int32_t seq_len, const lsa_heads *heads, int32_t block, float softmax_scale,
                                   void *out, int64_t *tile_counter, void *stream) {
    if (lsa_status s = check_kv(kv)) return s;
    if (lsa_status s = check_heads(heads, kv, true)) return s;
    PrefillArgs p{};
    bool empty = false;
    if (lsa_status s = prefill_setup(p, q, q_dtype, kv, page_table, seq_len, heads->num_q_heads, block,
                                     softmax_scale, out, tile_counter, empty))
        return s;
    if (empty) return ok();
    p.sink_blocks = heads->sink_blocks;
    p.local_blocks = heads->local_blocks;
    for (int i = 0; i < kv->num_kv_heads; ++i) {
        if (heads->head_kind[i] == LSA_RETRIEVAL_HEAD) p.ret_heads[p.n_ret++] = (uint8_t)i;
        else p.str_heads[p.n_str++] = (uint8_t)i;
    }
    // bf16 with one or two query heads per KV head: a work item takes 4 / G query tiles
    if (q_dtype == LSA_BF16 && (p.group == 1 || p.group == 2)) {
        p.q_tiles = 4 / p.group;
        p.n_qgroups = (p.n_qblocks + p.q_tiles - 1) / p.q_tiles;
        p.n_items = kv->num_kv_heads * p.n_qgroups * p.head_groups;
    }
    return from_hip(launch_prefill(p, q_dtype, (hipStream_t)stream), "prefill launch");
}

lsa_status lsa_sparse_prefill_attn_csr(const void *q, int32_t q_dtype, const lsa_kv *kv,
                                       const int32_t *page_table, int32_t seq_len, int32_t num_q_heads,
                                       int32_t block, const int32_t *row_ptr, const int32_t *col_idx,
                                       int32_t nnz, const int32_t *order, float softmax_scale, void *out,
                                       int64_t *tile_counter, void *stream) {
    if (lsa_status s = check_kv(kv)) return s;
    if (num_q_heads < 1 || num_q_heads % kv->num_kv_heads != 0)
        return fail(LSA_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                    num_q_heads, kv->num_kv_heads);
    if (num_q_heads / kv->num_kv_heads > 16)
        return fail(LSA_ERR_UNSUPPORTED, "GQA group size %d > 16", num_q_heads / kv->num_kv_heads);
    if (nnz < 0) return fail(LSA_ERR_INVALID_ARG, "nnz %d < 0", nnz);
    if (!row_ptr || (nnz > 0 && !col_idx)) return fail(LSA_ERR_INVALID_ARG, "row_ptr and col_idx must be non-NULL");
    PrefillArgs p{};
    bool empty = false;
    if (lsa_status s = prefill_setup(p, q, q_dtype, kv, page_table, seq_len, num_q_heads, block, softmax_scale, out,
                                     tile_counter, empty))
        return s;
    if (empty) return ok();
    // every KV head follows its own rows of the mask; work items are ordered like retrieval heads
    for (int i = 0; i < kv->num_kv_heads; ++i) p.ret_heads[p.n_ret++] = (uint8_t)i;
    // bf16 with one or two query heads per KV head: a work item takes 4 / G
    // query tiles and walks the union of their rows.  A work order then
    // starts with one code per group of query tiles (block_mask_schedule puts
    // them first), and only those leading entries are read.
    if (q_dtype == LSA_BF16 && mask_q_tiles(p.group, p.n_qblocks) > 1) {
        p.q_tiles = mask_q_tiles(p.group, p.n_qblocks);
        p.n_qgroups = (p.n_qblocks + p.q_tiles - 1) / p.q_tiles;
        p.n_items = kv->num_kv_heads * p.n_qgroups * p.head_groups;
    }
    p.row_ptr = row_ptr;
    p.col_idx = col_idx;
    p.nnz = nnz;
    p.order = order;
    return from_hip(launch_prefill(p, q_dtype, (hipStream_t)stream), "prefill launch");
}

lsa_status lsa_block_mask_schedule(const int32_t *row_ptr, int32_t num_kv_heads, int32_t num_q_heads,
                                   int32_t seq_len, int32_t block, int32_t *order) {
    if (block != 64) return fail(LSA_ERR_UNSUPPORTED, "block %d: only 64-token tiles are built", block);
    if (num_kv_heads < 1 || num_q_heads < 1 || num_q_heads % num_kv_heads != 0 || seq_len < 0)
        return fail(LSA_ERR_INVALID_ARG, "num_kv_heads %d, num_q_heads %d, seq_len %d", num_kv_heads, num_q_heads,
                    seq_len);
    if (!row_ptr || !order) return fail(LSA_ERR_INVALID_ARG, "row_ptr and order must be non-NULL");
    const int n = (seq_len + 63) / 64;
    const int G = num_q_heads / num_kv_heads;
    const int hg = (G + 3) / 4;
    // With query-tile groups (bf16, G <= 2) a work item covers QT tiles
    // n-1-QT*j-QT+1 .. n-1-QT*j; its cost follows the longest row of the
    // group.  The group's highest tile leads: leaders come first, then the
    // other codes, each part longest first, so a kernel that reads one code
    // per group and one that reads every code both find a balanced order.
    const int QT = mask_q_tiles(G, n);
    std::vector<std::pair<long long, int>> lead, rest;  // (sort key, item code)
    lead.reserve((size_t)num_kv_heads * n * hg);
    for (int h = 0; h < num_kv_heads; ++h) {
        const int32_t *rp = row_ptr + (size_t)h * (n + 1);
        for (int a = 0; a < n; ++a) {
            const bool leader = (n - 1 - a) % QT == 0;
            long long len = (long long)rp[a + 1] - rp[a];
            if (leader)
                for (int s = 1; s < QT && a - s >= 0; ++s) len = std::max(len, (long long)rp[a - s + 1] - rp[a - s]);
            for (int g = 0; g < hg; ++g) {
                const int code = (h * n + a) * hg + g;
                // longest first; among equal lengths, later query tiles first, then the code
                (leader ? lead : rest).push_back({-(len * ((long long)n + 1) + a), code});
            }
        }
    }
    const auto by_key = [](const std::pair<long long, int> &x, const std::pair<long long, int> &y) {
        return x.first < y.first;
    };
    std::stable_sort(lead.begin(), lead.end(), by_key);
    std::stable_sort(rest.begin(), rest.end(), by_key);
    size_t i = 0;
    for (const auto &e : lead) order[i++] = e.second;
    for (const auto &e : rest) order[i++] = e.second;
    return ok();
}

lsa_status lsa_check_block_mask(const int32_t *row_ptr, const int32_t *col_idx, int32_t num_kv_heads,
                                int32_t seq_len, int32_t block, int32_t nnz) {
    if (block != 64) return fail(LSA_ERR_UNSUPPORTED, "block %d: only 64-token tiles are built", block);
    if (num_kv_heads < 1 || seq_len < 0 || nnz < 0)
        return fail(LSA_ERR_INVALID_ARG, "num_kv_heads %d, seq_len %d, nnz %d", num_kv_heads, seq_len, nnz);
    if (!row_ptr || (nnz > 0 && !col_idx)) return fail(LSA_ERR_INVALID_ARG, "row_ptr and col_idx must be non-NULL");
    const int n = (seq_len + 63) / 64;
    for (int h = 0; h < num_kv_heads; ++h) {
        const int32_t *rp = row_ptr + (size_t)h * (n + 1);
        if (rp[0] < 0) return fail(LSA_ERR_INVALID_ARG, "head %d: row_ptr[0] = %d < 0", h, rp[0]);
        for (int a = 0; a < n; ++a) {
            if (rp[a + 1] < rp[a] || rp[a + 1] > nnz)
                return fail(LSA_ERR_INVALID_ARG, "head %d, query tile %d: row_ptr %d -> %d outside [.., %d]", h, a,
                            rp[a], rp[a + 1], nnz);
            for (int e = rp[a]; e < rp[a + 1]; ++e) {
                const int c = col_idx[e];
                if (c < 0 || c > a)
                    return fail(LSA_ERR_INVALID_ARG, "head %d, query tile %d: key tile %d outside [0, %d]", h, a, c, a);
                if (e > rp[a] && c <= col_idx[e - 1])
                    return fail(LSA_ERR_INVALID_ARG, "head %d, query tile %d: key tiles not strictly ascending", h, a);
            }
        }
    }
    return ok();
}

}  // extern "C"
