/*
 * lsa.h — C ABI of the MI355X (gfx950) block-sparse attention library with
 * hierarchical, query-aware KV page selection.
 *
 * Method sources (cited by page title and section):
 *   [LS-X] "MLSys 2025論文解説: LServe — 統一疎アテンションによる長文脈LLM推論の効率化",
 *          section 技術的詳細: 静的スパーシティ (retrieval / streaming heads,
 *          Lambda mask of sink + local tokens), 動的スパーシティ (the page score
 *          S^j = sum_i max(q[i] k_max^j[i], q[i] k_min^j[i])), 階層的ページング
 *          (physical page N_P = g * N_L logical pages; physical importance is the
 *          max of its logical pages' scores), 統一ブロックスパースアテンション
 *          (figure: one block-sparse kernel for both head kinds and phases;
 *          top-K physical pages at decode) and Reusable Page Selection (one
 *          selection serves k = 4 consecutive decode tokens).
 *   [LS-A] "LServe: Efficient Long-sequence LLM Serving with Unified Sparse
 *          Attention" (abstract page): streaming heads in prefill and decode; a
 *          constant number of KV pages regardless of context length.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked [host].
 *   - Every buffer is owned by the caller; the library allocates nothing and
 *     keeps no state of its own between calls (the one exception is the
 *     static scratch of lsa_sparse_decode_attn_noalloc).  Workspaces are sized by the
 *     *_workspace queries.  The selection and decode workspaces hold arrival
 *     counters that must be zero when a call starts; every completed call
 *     leaves them zero, so zero-filling a workspace once, before its first
 *     use, is enough.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise the host.
 *   - Arguments are validated on the host before any launch.  A validation
 *     failure returns a negative lsa_status, records a message readable with
 *     lsa_last_error() (thread-local) and launches nothing.  A failed launch
 *     returns LSA_ERR_HIP with the runtime's message.  No C++ exception
 *     crosses this boundary.
 *   - Device-side contents are trusted: page ids outside [0, num_pages),
 *     seq_lens above max_pages * page_size or selected pages beyond the
 *     sequence are undefined behaviour.
 *   - Supported shapes: head_dim 64 or 128; page_size in {16, 32, 64, 128,
 *     256} and a multiple of logical_page; logical_page in {8, 16, 32, 64};
 *     num_q_heads a multiple of num_kv_heads with group size
 *     G = num_q_heads / num_kv_heads <= 16.  Query head h uses KV head h / G.
 *
 * Paged KV pool layout (caller-owned, fixed).  A page holds page_size tokens
 * of one KV head as page_size/BT blocks of BT consecutive tokens, BT =
 * min(page_size, 32) (one block of 16 tokens for 16-token pages); inside a
 * block, keys are tiles of BT tokens x 32 channels and values are
 * channel-major rows of BT tokens:
 *   K, f32/bf16:  [num_pages][H_kv][page_size/BT][head_dim/32][BT][32]
 *                 key (token p, channel c) of a page at
 *                 [p/BT][c/32][p%BT][c%32]
 *   V, f32/bf16:  [num_pages][H_kv][page_size/BT][head_dim][BT]
 *                 value (p, c) at [p/BT][c][p%BT]
 *   K, int4:      [num_pages][H_kv][page_size/BT][head_dim/32][BT][16] bytes:
 *                 the K tile with channels 2i, 2i+1 of a tile row packed in
 *                 byte i (2i in the low nibble)
 *   V, int4:      [num_pages][H_kv][page_size/BT][head_dim][BT/2] bytes: the
 *                 V rows with tokens 2j, 2j+1 packed in byte j (2j low nibble)
 *   k_sz, v_sz:   int4 only, [num_pages][H_kv][2] IEEE fp16 {scale s, zero z},
 *                 s > 0; a stored code c means (c - z) * s.
 *   Every 16-byte group a kernel loads is a run of one tile row, so the
 *   matrix-core operands of a 16-token group of keys or values are single
 *   contiguous 1 KiB reads.
 *   Token p of sequence b is slot p % page_size of pool page
 *   page_table[b * max_pages + p / page_size].
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lsa_status;
#define LSA_OK                0
#define LSA_ERR_INVALID_ARG  (-1)
#define LSA_ERR_UNSUPPORTED  (-2)
#define LSA_ERR_WORKSPACE    (-3)
#define LSA_ERR_HIP          (-4)

#define LSA_F32   0
#define LSA_BF16  1
#define LSA_INT4  2

#define LSA_RETRIEVAL_HEAD 0
#define LSA_STREAMING_HEAD 1

/* How the page scores of the query heads that share one KV head combine
 * (lsa_heads.score_aggregation): their sum (the default), or their maximum. */
#define LSA_AGG_SUM 0
#define LSA_AGG_MAX 1

/* [host] descriptor of the constant-size cache of the streaming heads
 * ([LS-X] 静的スパーシティ: a streaming head only ever attends its sink and
 * its most recent tokens, so its cost, and here its memory, does not grow with
 * the context).  For every sequence b and streaming KV head (H_s of them,
 * numbered s = 0 .. H_s - 1 in KV-head order) the cache holds sink_pages +
 * ring_pages pages of page_size tokens in the pool's page layout:
 *   K, V:        [B][H_s][sink_pages + ring_pages] pages, each laid out as one
 *                (pool page, KV head) of the paged pool (layout above);
 *   k_sz, v_sz:  int4 only, [B][H_s][sink_pages + ring_pages][2] fp16 {s, z}.
 * Sequence page m (tokens m*N_P .. m*N_P + N_P - 1) of (b, s) is cache page
 *   m                                          if m < sink_pages,
 *   sink_pages + (m - sink_pages) % ring_pages otherwise,
 * so the ring keeps the ring_pages most recent pages past the sink.  With
 * sink_pages >= ceil(sink_tokens / N_P) and ring_pages >= ceil(local_tokens /
 * N_P) + 1 (lsa_stream_cache_pages) every token a streaming head attends is
 * in the cache.  Its size is independent of the context length. */
typedef struct lsa_stream_cache {
    int32_t sink_pages;     /* pages kept from the start of each sequence           */
    int32_t ring_pages;     /* pages of the ring of recent pages                    */
    void *k;                /* K pages                                              */
    void *v;                /* V pages                                              */
    uint16_t *k_sz;         /* int4 only, else NULL                                 */
    uint16_t *v_sz;         /* int4 only, else NULL                                 */
} lsa_stream_cache;

/* [host] descriptor of the paged KV pool (layout above). */
typedef struct lsa_kv {
    int32_t kv_dtype;       /* LSA_F32 | LSA_BF16 | LSA_INT4                      */
    int32_t num_kv_heads;   /* H_kv                                               */
    int32_t head_dim;       /* D: 64 or 128                                       */
    int32_t page_size;      /* N_P, tokens per physical page                      */
    int32_t logical_page;   /* N_L, tokens per logical page; N_P = g * N_L        */
    int32_t reserved;       /* must be 0                                          */
    int64_t num_pages;      /* pool capacity P                                    */
    const void *k;          /* K pool                                             */
    const void *v;          /* V pool                                             */
    const uint16_t *k_sz;   /* int4 only, else NULL                               */
    const uint16_t *v_sz;   /* int4 only, else NULL                               */
    /* NULL: every KV head lives in the pool ([P][H_kv] pages, as above).
     * Non-NULL: the pool pages hold only the retrieval heads, [P][H_r] with
     * the H_r retrieval heads in KV-head order (the statistics pool likewise),
     * and the streaming heads live in this cache.  A pool of this kind needs
     * the head classification (lsa_heads) in every call, and prefill, which
     * reads every head, does not take it. */
    const lsa_stream_cache *stream_cache;
} lsa_kv;

/* [host] descriptor of a decode batch. */
typedef struct lsa_seqs {
    int32_t batch;              /* B                                              */
    int32_t max_pages;          /* row stride of page_table                       */
    const int32_t *page_table;  /* [B][max_pages] pool page id of sequence page m */
    const int32_t *seq_lens;    /* [B] tokens in cache, the current one included;
                                   each in [1, max_pages * page_size]             */
} lsa_seqs;

/* [host] head classification ([LS-X] 静的スパーシティ: a head is either a
 * retrieval head or a streaming head; the class is fixed per KV head and known
 * when the model is loaded). */
typedef struct lsa_heads {
    const uint8_t *head_kind;   /* [host] [H_kv]: LSA_RETRIEVAL_HEAD | LSA_STREAMING_HEAD */
    int32_t num_q_heads;        /* H_q, a multiple of H_kv                        */
    int32_t sink_tokens;        /* decode Lambda: tokens p < sink_tokens ...      */
    int32_t local_tokens;       /* ... or t - p < local_tokens are attended       */
    int32_t sink_blocks;        /* prefill Lambda, in tiles: tiles c < sink_blocks */
    int32_t local_blocks;       /* ... or a - c < local_blocks (diagonal counts)  */
    int32_t score_aggregation;  /* LSA_AGG_SUM (0) or LSA_AGG_MAX: how the G heads'
                                   page scores combine in lsa_select_pages        */
} lsa_heads;

/* Bytes of the logical-page statistics pool that matches `kv`:
 *   f32/bf16: [num_pages][H][g][2][head_dim] elements of kv_dtype
 *             (index 0 = channel minimum, 1 = channel maximum), g = N_P / N_L;
 *   int4:     [num_pages][H][g][head_dim] bytes, byte = c_min | c_max << 4;
 * H = H_kv, or the number of retrieval heads when kv->stream_cache is set
 * (pass their count in `heads`; NULL heads means every head is in the pool).
 * Source: [LS-X] 動的スパーシティ and 階層的ページング (channel-wise k_min /
 * k_max per logical page, kept beside each physical page). */
lsa_status lsa_page_stats_bytes(const lsa_kv *kv, const lsa_heads *heads /* nullable */,
                                size_t *bytes /* [host] out */);

/* The smallest streaming-head cache for these shapes: *sink_pages =
 * ceil(sink_tokens / N_P) and *ring_pages = ceil(local_tokens / N_P) + 1 (the
 * local window of a token spans at most that many pages).  Source: [LS-X]
 * 静的スパーシティ (sink + local tokens of a streaming head). */
lsa_status lsa_stream_cache_pages(const lsa_kv *kv, const lsa_heads *heads, int32_t *sink_pages /* [host] out */,
                                  int32_t *ring_pages /* [host] out */);

/* Fill a streaming-head cache from a paged pool that holds every head (src,
 * stream_cache NULL): for every sequence b, with tokens 0 .. seq_lens[b] - 1
 * in src, each cache page receives the whole src page it stands for (the sink
 * pages, and the ring_pages most recent pages past them; pages past the
 * sequence are left untouched), int4 scale and zero point included.  This is
 * the hand-over after a prefill over a full pool.  cache: the destination,
 * shapes as in lsa_stream_cache. */
lsa_status lsa_stream_cache_fill(const lsa_kv *src, const lsa_seqs *seqs, const lsa_heads *heads,
                                 const lsa_stream_cache *cache, void *stream);

/* Append the key and value of the newest token t = seq_lens[b] - 1 of every
 * sequence b, for every KV head ([LS-X] Reusable Page Selection: a decode step
 * appends its token's K/V before selecting and attending).  Retrieval heads
 * (and streaming heads when kv->stream_cache is NULL) are written to slot
 * t % N_P of pool page page_table[b][t / N_P]; streaming heads go to their
 * cache page when kv->stream_cache is set.
 * k_new, v_new: [B][H_kv][head_dim] of kv_dtype (f32 / bf16), or for int4 the
 * codes [B][H_kv][head_dim / 2] bytes (channel 2i in the low nibble of byte i)
 * with k_new_sz, v_new_sz: [B][H_kv][2] fp16 {s, z} of the token's page,
 * written to the page's entry (every token of a page shares it).
 * stats: NULL, or the statistics pool: the statistics of the logical page that
 * holds t are updated for every retrieval head (a new logical page starts
 * from the token; otherwise the minimum / maximum take the token in), which
 * is what lsa_build_page_stats(first_token = t) computes, so a decode step
 * then needs no statistics refresh in lsa_sparse_decode_attn (stats NULL).
 * One kernel launch. */
lsa_status lsa_append_kv(const lsa_kv *kv, const lsa_seqs *seqs, const lsa_heads *heads, const void *k_new,
                         const void *v_new, const uint16_t *k_new_sz, const uint16_t *v_new_sz, void *stats,
                         void *stream);

/* Build the channel-wise min / max of the keys of logical pages
 * ([LS-X] 動的スパーシティ: statistics of logical page j; 階層的ページング:
 * N_L-token logical pages inside N_P-token physical pages).
 *
 * For every sequence b and KV head (only retrieval heads when `heads` is not
 * NULL; every head when it is NULL) the logical pages j that overlap
 * [first_token[b], seq_lens[b]) are recomputed from their valid tokens
 * [j*N_L, min((j+1)*N_L, seq_lens[b])).  Logical pages with no valid token are
 * left untouched.  first_token == NULL means 0 for every sequence (a full
 * build after a prefill).  max_new_tokens [host] bounds seq_lens[b] -
 * first_token[b] over the batch (it sizes the launch; 1 for a decode step);
 * 0 means max_pages * page_size.  Min and max are exact (no rounding).
 * stats: the statistics pool, layout as in lsa_page_stats_bytes.
 * Call after the K rows of the new tokens are in the pool. */
lsa_status lsa_build_page_stats(const lsa_kv *kv, const lsa_seqs *seqs,
                                const lsa_heads *heads, const int32_t *first_token,
                                int32_t max_new_tokens, void *stats, void *stream);

/* Workspace of lsa_select_pages, in bytes. */
lsa_status lsa_select_pages_workspace(const lsa_kv *kv, const lsa_seqs *seqs,
                                      const lsa_heads *heads, size_t *bytes /* [host] out */);

/* Query-aware top-K physical page selection with reuse
 * ([LS-X] 動的スパーシティ, 階層的ページング, the figure's top-K physical pages,
 * Reusable Page Selection; [LS-A] constant page budget).
 *
 * Runs only when decode_step % reuse_interval == 0; otherwise returns LSA_OK
 * and leaves `selected` unchanged (the previous selection is reused).  For
 * each sequence b and retrieval KV head kv, with the group's queries
 * q_h (h = kv*G .. kv*G+G-1):
 *   S_h^j = sum_i max(q_h[i] * kmax^j[i], q_h[i] * kmin^j[i])   for every
 *          logical page j holding a valid token;
 *   S^j  = sum_h S_h^j (heads->score_aggregation == LSA_AGG_SUM, the default)
 *          or max_h S_h^j (LSA_AGG_MAX);
 *   P_m  = max over the logical pages j of physical page m (j / g == m);
 *   selected[b][kv][0..K-1] = the K = token_budget / page_size pages m of
 *          largest P_m, ties to the lower m, in ascending m, padded with -1
 *          when the sequence has fewer than K pages.
 * Products are exact and S^j, P_m are accumulated and compared in fp64.
 * The logical page that holds the current token t = seq_lens[b] - 1 is scored
 * from its keys in the pool (min / max of tokens j*N_L .. t taken on the fly),
 * so its entry in `stats` may be stale; every earlier logical page is read
 * from `stats`.
 * Streaming heads' rows of `selected` are not written.
 * q: [B][H_q][head_dim] of q_dtype (LSA_F32 or LSA_BF16).
 * stats: as built by lsa_build_page_stats for tokens < seq_lens[b].
 * selected: [B][H_kv][K] int32.
 * workspace: at least lsa_select_pages_workspace bytes, 256-byte aligned,
 * zero-filled before its first use: its leading B * H_kv int32 arrival
 * counters must be zero when a call starts, and each completed call leaves
 * them zero; calls that share a workspace must not overlap in time.
 * Up to 4096 pages per sequence one kernel is launched (the last score
 * workgroup of a (sequence, head) runs its top-K); above that a second,
 * top-K kernel follows. */
lsa_status lsa_select_pages(const void *q, int32_t q_dtype, const lsa_kv *kv,
                            const void *stats, const lsa_seqs *seqs,
                            const lsa_heads *heads, int32_t token_budget,
                            int32_t decode_step, int32_t reuse_interval,
                            int32_t *selected, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Workspace of lsa_sparse_decode_attn, in bytes. */
lsa_status lsa_decode_workspace(const lsa_kv *kv, const lsa_seqs *seqs,
                                const lsa_heads *heads, int32_t token_budget,
                                size_t *bytes /* [host] out */);

/* Block-sparse paged decode attention for retrieval and streaming heads
 * ([LS-X] 静的スパーシティ, the figure's unified block-sparse kernel;
 * [LS-A] constant KV page count per step).
 *
 * For each sequence b, t = seq_lens[b] - 1, and query head h (KV head
 * kv = h / G):
 *   retrieval kv: attended keys A = { p <= t : p / N_P in selected[b][kv] or
 *                 p / N_P == t / N_P }  (the current page is always read);
 *   streaming kv: A = { p <= t : p < sink_tokens or t - p < local_tokens };
 *   out[b][h] = sum_{p in A} softmax_p(scale * q_h . k_p) v_p.
 * Only the pages that intersect A are read; a K/V page read serves all G
 * query heads of its group.
 * q, out: [B][H_q][head_dim]; supported (q_dtype, kv_dtype) pairs are
 * (LSA_F32, LSA_F32), (LSA_BF16, LSA_BF16) and (LSA_BF16, LSA_INT4); out has
 * q's dtype (round to nearest even).  Accumulation is fp32.
 * selected: [B][H_kv][K] as written by lsa_select_pages (rows of streaming
 * heads are not read; may be NULL when every head is a streaming head).
 * softmax_scale: 0 means 1 / sqrt(head_dim).
 * stats: NULL, or the statistics pool of lsa_build_page_stats: the call then
 * also refreshes, for every retrieval head, the statistics of the logical page
 * that holds token t (what lsa_build_page_stats does with first_token = t), so
 * a decode step needs no separate statistics launch.
 * workspace: at least lsa_decode_workspace bytes, 256-byte aligned, zero-filled
 * before its first use (its leading B * H_kv int32 arrival counters must be
 * zero when a call starts; each completed call leaves them zero); calls that
 * share a workspace must not overlap in time (same stream, or ordered).
 * One kernel is launched: the split-KV pass, whose last workgroup per
 * (sequence, KV head) merges the partial results in chunk order. */
lsa_status lsa_sparse_decode_attn(const void *q, int32_t q_dtype, const lsa_kv *kv,
                                  const lsa_seqs *seqs, const lsa_heads *heads,
                                  const int32_t *selected, int32_t token_budget,
                                  float softmax_scale, void *out, void *stats,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* lsa_sparse_decode_attn without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It computes exactly what
 * lsa_sparse_decode_attn computes, with the same kernels, and allocates
 * nothing: its scratch (the arrival counters and the split-KV partial
 * records that lsa_decode_workspace sizes) is a 16 MiB (16777216-byte)
 * static device array inside the library, one copy per GPU, held until the
 * process ends.  The copy of the current device (hipGetDevice) is used; its
 * address is looked up on the first call on that device.  A batch whose
 * lsa_decode_workspace size exceeds 16 MiB is rejected with
 * LSA_ERR_UNSUPPORTED and nothing is launched (config-2-shaped layers, 8 x 8
 * heads at a 4096-token budget, need 1.25 MB; 64 x 8 heads at N_P = 128 need
 * 10 MB).  Each call first clears the counters with a small fill kernel on
 * `stream`, then launches the decode kernel.  Every call on a GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and give undefined results; order them on one stream.
 * Arguments and errors are otherwise those of lsa_sparse_decode_attn. */
lsa_status lsa_sparse_decode_attn_noalloc(const void *q, int32_t q_dtype, const lsa_kv *kv,
                                          const lsa_seqs *seqs, const lsa_heads *heads,
                                          const int32_t *selected, int32_t token_budget,
                                          float softmax_scale, void *out, void *stats, void *stream);

/* Workspace of lsa_decode_step, in bytes: the larger of
 * lsa_select_pages_workspace and lsa_decode_workspace. */
lsa_status lsa_decode_step_workspace(const lsa_kv *kv, const lsa_seqs *seqs, const lsa_heads *heads,
                                     int32_t token_budget, size_t *bytes /* [host] out */);

/* One whole decode step of every sequence b, t = seq_lens[b] - 1 being the
 * newest token ([LS-X] Reusable Page Selection: a step appends the token's
 * K/V, selects pages (every reuse_interval steps) and attends; 動的スパーシティ
 * and 階層的ページング for the selection; 統一ブロックスパースアテンション for the
 * attention).  Its results are those of
 *   lsa_append_kv(kv, seqs, heads, k_new, v_new, k_new_sz, v_new_sz, stats);
 *   lsa_select_pages(q, q_dtype, kv, stats, seqs, heads, token_budget,
 *                    decode_step, reuse_interval, selected);
 *   lsa_sparse_decode_attn(q, q_dtype, kv, seqs, heads, selected,
 *                          token_budget, softmax_scale, out, stats = NULL);
 * in two launches instead of three: the selection takes token t's key row
 * (and int4 page scale / zero point) from k_new (k_new_sz) instead of the
 * pool, and the decode kernel's workgroup that reads t's page attends t from
 * the staged rows and writes them to the pool or the stream cache (and, for
 * retrieval heads, folds t into its logical page's statistics), so the token
 * does not make a round trip through memory before it is attended.
 * Arguments are those of the three calls; stats must be non-NULL when a
 * retrieval head exists.  selected may be NULL only when every head is a
 * streaming head.  workspace: at least lsa_decode_step_workspace bytes,
 * 256-byte aligned, zero-filled before its first use, with the counter
 * contract of lsa_select_pages and lsa_sparse_decode_attn (both launches use
 * it in stream order).  The pool slots of token t and the statistics of its
 * logical page may be read and written by this call only: calls on other
 * streams that read them race.  Errors: those of the three calls, all
 * checked before anything is launched. */
lsa_status lsa_decode_step(const void *q, int32_t q_dtype, const lsa_kv *kv, const lsa_seqs *seqs,
                           const lsa_heads *heads, const void *k_new, const void *v_new,
                           const uint16_t *k_new_sz, const uint16_t *v_new_sz, void *stats,
                           int32_t token_budget, int32_t decode_step, int32_t reuse_interval,
                           int32_t *selected, float softmax_scale, void *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Block-sparse causal prefill attention of one sequence over non-empty tiles
 * only ([LS-X] 統一ブロックスパースアテンション: iterate the non-empty blocks;
 * the figure's retrieval heads use a static causal pattern in prefill and
 * streaming heads sink + local blocks; speed-up 1/(1-r)).
 *
 * Tiles are block x block tokens (block must be 64).  Query tile a sees key
 * tile c when c <= a and (retrieval head, or c < sink_blocks, or
 * a - c < local_blocks); inside a visible tile, key p is seen by query t iff
 * p <= t.  out[t][h] = softmax over the visible keys of scale * q.k, times v.
 * q, out: [seq_len][H_q][head_dim]; (q_dtype, kv_dtype) is (LSA_BF16, LSA_BF16)
 * or (LSA_F32, LSA_F32) with head_dim 64 (the f32 path is the small-model
 * path).  page_table: [ceil(seq_len / page_size)] pool page
 * ids of the sequence; page_size must be a multiple of 64.
 * tile_counter: NULL, or an int64 to which the number of (query head, tile)
 * pairs computed is added (it equals the non-empty tile count of the mask).
 * softmax_scale: 0 means 1 / sqrt(head_dim). */
lsa_status lsa_sparse_prefill_attn(const void *q, int32_t q_dtype, const lsa_kv *kv,
                                   const int32_t *page_table, int32_t seq_len,
                                   const lsa_heads *heads, int32_t block,
                                   float softmax_scale, void *out,
                                   int64_t *tile_counter, void *stream);

/* Block-sparse causal prefill attention of one sequence under an arbitrary
 * static block mask given as per-KV-head CSR lists of key tiles ([LS-X]
 * 統一ブロックスパースアテンション: an iterator over the non-empty blocks of a
 * static pattern, cost falling as 1/(1-r); 主要な貢献: iterator-based
 * block-sparse kernels).
 *
 * Tiles are block x block tokens (block must be 64); n = ceil(seq_len / 64).
 * row_ptr: [device] int32 [num_kv_heads][n + 1]; the key tiles of query tile a
 * for KV head kv are col_idx[row_ptr[kv][a] .. row_ptr[kv][a + 1]), offsets
 * into col_idx of nnz int32 entries ([device]).  A valid mask has
 * 0 <= row_ptr[kv][0] <= ... <= row_ptr[kv][n] <= nnz and, within a row, key
 * tiles strictly ascending in [0, a]; lsa_check_block_mask validates a host
 * copy.  The kernels clamp offsets to [0, nnz] and tiles to [0, a], so a
 * malformed mask gives unspecified outputs but no access outside the arrays.
 * Inside a listed tile, key p is seen by query t iff p <= t; a query tile
 * with an empty row gets zero output.  The query heads of a KV head share its
 * rows.  q, out, page_table, dtypes, softmax_scale and tile_counter are as for
 * lsa_sparse_prefill_attn (the counter adds (row length) x G per row).
 * With bf16 q and G <= 2 (and n <= 4096) one workgroup takes QT = 4 / G
 * query tiles n-1-QT*j-QT+1 .. n-1-QT*j and walks the union of their rows.
 * order: NULL, or [device] int32 [num_kv_heads * n * ceil(G / 4)], the work
 * order written by lsa_block_mask_schedule for this mask and these head
 * counts (entries are clamped to the item range).  Workgroups start in this
 * order, round robin over the XCDs, so rows of equal length side by side keep
 * every XCD busy; a mask whose rows differ in length runs up to twice as fast
 * with it.  Where QT > 1 only the first num_kv_heads * ceil(n / QT) entries
 * are read, each standing for the group of query tiles that holds its tile;
 * another permutation than the schedule's may then leave groups out. */
lsa_status lsa_sparse_prefill_attn_csr(const void *q, int32_t q_dtype, const lsa_kv *kv,
                                       const int32_t *page_table, int32_t seq_len,
                                       int32_t num_q_heads, int32_t block,
                                       const int32_t *row_ptr, const int32_t *col_idx,
                                       int32_t nnz, const int32_t *order, float softmax_scale,
                                       void *out, int64_t *tile_counter, void *stream);

/* Work order of a static block mask for lsa_sparse_prefill_attn_csr, computed
 * once per mask on the host: row_ptr is a [host] copy ([num_kv_heads][n + 1]);
 * order ([host] out, num_kv_heads * n * ceil(G / 4) int32) receives every work
 * item (kv * n + a) * ceil(G / 4) + g once, longest rows first, then later
 * query tiles first.  At G <= 2 (n <= 4096) the codes of each query-tile
 * group's highest tile come first, ranked by the longest row of the group,
 * then the other codes, so the same order serves the bf16 kernel (which
 * reads one code per group) and the f32 kernel (which reads them all). */
lsa_status lsa_block_mask_schedule(const int32_t *row_ptr, int32_t num_kv_heads,
                                   int32_t num_q_heads, int32_t seq_len, int32_t block,
                                   int32_t *order);

/* Host-side check of a block mask for lsa_sparse_prefill_attn_csr: row_ptr
 * and col_idx are [host] copies with the layout above.  Returns LSA_OK, or
 * LSA_ERR_INVALID_ARG naming the first bad head / query tile. */
lsa_status lsa_check_block_mask(const int32_t *row_ptr, const int32_t *col_idx,
                                int32_t num_kv_heads, int32_t seq_len, int32_t block,
                                int32_t nnz);

/* Message of the last failed call on this thread ("" if none); never NULL. */
const char *lsa_last_error(void);

/* Library version string, "lsa <version> gfx950 src <sha>", with the first 16
 * hex digits of the SHA-256 of the sources the library was built from. */
const char *lsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
