// Internal declarations shared by the HIP translation units of liblsa.
// Not part of the public ABI (include/lsa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa.h"

namespace lsa {

constexpr int kMaxKvHeads = 64;   // H_kv limit (the head kinds travel as a 64-bit mask)
constexpr int kWave = 64;         // CDNA wavefront width
constexpr int kMaxDecodeChunks = 128;   // split-KV chunks per (sequence, KV head)

// Split-KV geometry of decode attention.  The MFMA path runs kDecodeWaves
// wavefronts per workgroup, each streaming up to 128 tokens (one page when
// pages are longer); the f32 path runs four wavefronts of one page each.  A
// workgroup takes one chunk of the attended page list: up to
// decode_chunk_pages pages, fewer when that spreads a launch that fits the
// chip in one round more evenly over the CUs (the decode geometry on the
// host); wavefront w takes the chunk's pages PPW*w .. PPW*w + PPW - 1.
constexpr int kDecodeWaves = 4;
constexpr int kMaxChunkPages = 32;
constexpr int kDecodeWaveTokens = 128;
// XCDs of the part; workgroups are handed to them round robin in number order
constexpr int kXcds = 8;
// Static-mask prefill with several query tiles per workgroup builds the union
// of their rows in LDS: rows of up to this many 64-token tiles
constexpr int kPrefillMaxUnionTiles = 4096;
// Query tiles per static-mask work item in the bf16 kernel: four wavefront
// pairs cover G query heads x (4 / G) query tiles when G is 1 or 2.
__host__ __device__ constexpr int mask_q_tiles(int group, int n_qblocks) {
    return group <= 2 && n_qblocks <= kPrefillMaxUnionTiles ? 4 / group : 1;
}
__host__ __device__ constexpr int decode_pages_per_wave(int kv_dtype, int page_size) {
    return kv_dtype == LSA_F32 || page_size >= kDecodeWaveTokens ? 1 : kDecodeWaveTokens / page_size;
}
__host__ __device__ constexpr int decode_chunk_pages(int kv_dtype, int page_size) {
    return kv_dtype == LSA_F32 ? 4 : kDecodeWaves * decode_pages_per_wave(kv_dtype, page_size);
}
// Wavefronts per SIMD the MFMA decode kernel's register budget is set for:
// three for the int4 instances with 64- and 128-token pages (at most 168
// VGPRs: past that, with the allocation granule of 8, a SIMD holds two, and a
// launch of 768 workgroups, B = 16 at a 4096-token budget, no longer fits the
// chip in one round), two otherwise (the 16- and 32-token int4 instances
// spill at 168).  With four wavefronts per workgroup this is also the
// workgroups per CU.
__host__ __device__ constexpr int decode_waves_per_simd(int kvt, int np) {
    return kvt == LSA_INT4 && (np == 64 || np == 128) ? 3 : 2;
}
constexpr int kComputeUnits = 256;        // CUs of the part (MI355X)
// split-KV records the last workgroup of a (sequence, KV head) loads per
// memory round trip when it merges them
constexpr int kDecodeMergeBatch = 12;

// ----------------------------------------------------------------------------
// numeric helpers (device)
// ----------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite here)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// IEEE binary16 bits -> float (exact)
__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return float(v);
}

// 2^x on the hardware exponential unit
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Loads of data read once per launch (decode K/V blocks, page statistics in
// scoring) carry the non-temporal hint, so the stream does not displace lines
// the rest of the launch still uses.
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4 *>(p)));
}
__device__ __forceinline__ uint2 load_stream8(const void *p) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint2, __builtin_nontemporal_load(static_cast<const u32x2 *>(p)));
}
__device__ __forceinline__ uint32_t load_stream4(const void *p) {
    return __builtin_nontemporal_load(static_cast<const uint32_t *>(p));
}

// Raw buffer resources (gfx9 family: dword 3 selects the 32-bit data format).
// A load through one takes its base from scalar registers and its lane offset
// from one VGPR, so a kernel that forms the lane offsets once issues its loads
// with no per-load vector address arithmetic.  The hardware range check
// covers the lane offset (plus the instruction's immediate): a lane whose
// offset is at or past `bytes` reads zeros; the scalar offset is not checked,
// so callers keep base + soff + voff inside the object themselves.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNt = 2;                      // the non-temporal hint of load_stream*
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kBufferWord3);
}
__device__ __forceinline__ uint4 buffer_stream16(const void *base, int bytes, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(base, bytes), voff, soff,
                                                                            kBufferNt));
}
__device__ __forceinline__ uint2 buffer_stream8(const void *base, int bytes, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(buffer_rsrc(base, bytes), voff, soff,
                                                                           kBufferNt));
}
__device__ __forceinline__ uint32_t buffer_stream4(const void *base, int bytes, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(base, bytes), voff, soff, kBufferNt);
}

// ----------------------------------------------------------------------------
// page layout: a page of N_P tokens of one KV head is a run of blocks of BT =
// min(N_P, 32) tokens (N_P/32 blocks of 32, or one block of 16 for 16-token
// pages); keys are [block][D/32][BT tokens][32 channels] tiles, values are
// [block][D][BT tokens] rows.  Offsets are in elements (int4: halve for the
// byte of an even channel / token).  bs = log2(BT).
// ----------------------------------------------------------------------------
__host__ __device__ constexpr int block_shift(int page_size) { return page_size < 32 ? 4 : 5; }
__device__ __forceinline__ size_t key_offset(int s, int c, int D, int bs = 5) {
    return (((size_t)(s >> bs) * (D >> 5) + (c >> 5)) << (bs + 5)) + (size_t)(s & ((1 << bs) - 1)) * 32 + (c & 31);
}
__device__ __forceinline__ size_t value_offset(int s, int c, int D, int bs = 5) {
    return (((size_t)(s >> bs) * D + c) << bs) + (s & ((1 << bs) - 1));
}

// ----------------------------------------------------------------------------
// cross-lane primitives on the VALU (DPP and gfx950 permlane swaps).  A
// ds_bpermute (what __shfl_* lowers to) goes through the LDS crossbar and
// costs a long round trip; chains of them dominated the small kernels.
// ----------------------------------------------------------------------------

// {x[l], x[l ^ 32]} in some order, in every lane l
__device__ __forceinline__ void pair32(uint32_t x, uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
}
// {x[l], x[l ^ 16]} in some order, in every lane l
__device__ __forceinline__ void pair16(uint32_t x, uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = r[0];
    b = r[1];
}
// a's lanes 32-63 trade places with b's lanes 0-31
__device__ __forceinline__ void swap_halves32(uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
// a's odd 16-lane rows (lanes 16-31, 48-63) trade places with b's even rows (0-15, 32-47)
__device__ __forceinline__ void swap_rows16(uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ float max_xor32(float x) {
    uint32_t a, b;
    pair32(__float_as_uint(x), a, b);
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float max_xor16(float x) {
    uint32_t a, b;
    pair16(__float_as_uint(x), a, b);
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float sum_xor32(float x) {
    uint32_t a, b;
    pair32(__float_as_uint(x), a, b);
    return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float sum_xor16(float x) {
    uint32_t a, b;
    pair16(__float_as_uint(x), a, b);
    return __uint_as_float(a) + __uint_as_float(b);
}

// DPP controls
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror
constexpr int kDppRowRor4 = 0x124;     // row_ror:4
constexpr int kDppRowRor8 = 0x128;     // row_ror:8

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const unsigned long long u = __double_as_longlong(v);
    const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xf, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

// Minimum (MAX = false) or maximum of v over aligned groups of N lanes (N = 1,
// 2, 4, 8, 16), result in every lane of the group.
template <int N, bool MAX>
__device__ __forceinline__ int group_minmax_i(int v) {
    auto op = [](int x, int y) { return MAX ? max(x, y) : min(x, y); };
    if constexpr (N >= 2) v = op(v, (int)dpp_u<kDppQuadSwap1>((uint32_t)v));
    if constexpr (N >= 4) v = op(v, (int)dpp_u<kDppQuadSwap2>((uint32_t)v));
    if constexpr (N >= 8) v = op(v, (int)dpp_u<kDppHalfMirror>((uint32_t)v));
    if constexpr (N >= 16) v = op(v, (int)dpp_u<kDppMirror>((uint32_t)v));
    return v;
}

// Sum of v over aligned groups of N lanes (N = 1, 2, 4, 8, 16, 32), result in every lane of the group.
template <int N>
__device__ __forceinline__ double group_sum_d(double v) {
    if constexpr (N >= 2) v += dpp_d<kDppQuadSwap1>(v);
    if constexpr (N >= 4) v += dpp_d<kDppQuadSwap2>(v);
    if constexpr (N >= 8) v += dpp_d<kDppHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_d<kDppMirror>(v);
    if constexpr (N >= 32) {
        const unsigned long long u = __double_as_longlong(v);
        uint32_t l0, l1, h0, h1;
        pair16((uint32_t)u, l0, l1);
        pair16((uint32_t)(u >> 32), h0, h1);
        v = __longlong_as_double((long long)(((unsigned long long)h0 << 32) | l0)) +
            __longlong_as_double((long long)(((unsigned long long)h1 << 32) | l1));
    }
    return v;
}

// max / sum over all 64 lanes of a wavefront, result in every lane
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __uint_as_float(dpp_u<kDppQuadSwap1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u<kDppQuadSwap2>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u<kDppHalfMirror>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u<kDppMirror>(__float_as_uint(v))));
    return max_xor32(max_xor16(v));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += __uint_as_float(dpp_u<kDppQuadSwap1>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u<kDppQuadSwap2>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u<kDppHalfMirror>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u<kDppMirror>(__float_as_uint(v)));
    return sum_xor32(sum_xor16(v));
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

// Bitwise and / or of a 64-bit value over the wavefront (every lane gets it).
__device__ __forceinline__ void wave_and_or(unsigned long long &a, unsigned long long &o) {
    uint32_t al = (uint32_t)a, ah = (uint32_t)(a >> 32), ol = (uint32_t)o, oh = (uint32_t)(o >> 32);
#define LSA_AO_STEP(C)                                                                  \
    al &= dpp_u<C>(al); ah &= dpp_u<C>(ah); ol |= dpp_u<C>(ol); oh |= dpp_u<C>(oh);
    LSA_AO_STEP(kDppQuadSwap1)
    LSA_AO_STEP(kDppQuadSwap2)
    LSA_AO_STEP(kDppHalfMirror)
    LSA_AO_STEP(kDppMirror)
#undef LSA_AO_STEP
    uint32_t x, y;
    pair16(al, x, y); al = x & y;
    pair16(ah, x, y); ah = x & y;
    pair16(ol, x, y); ol = x | y;
    pair16(oh, x, y); oh = x | y;
    pair32(al, x, y); al = x & y;
    pair32(ah, x, y); ah = x & y;
    pair32(ol, x, y); ol = x | y;
    pair32(oh, x, y); oh = x | y;
    a = ((unsigned long long)ah << 32) | al;
    o = ((unsigned long long)oh << 32) | ol;
}

// ----------------------------------------------------------------------------
// launch arguments
// ----------------------------------------------------------------------------

// The layer's KV heads as the kernels see them: the streaming heads as a bit
// mask (bit kv set: KV head kv is a streaming head), and where each head's
// pages sit in the pool: pool page p, head slot s of pool_heads, at element
// ((p * pool_heads + s) * N_P * D).  The pool holds every KV head (slot kv)
// or, when the streaming heads live in a stream cache, only the retrieval
// heads (slot = the head's rank among them).  Kernels take a head's kind,
// slot and rank from the mask with scalar bit operations: a per-head table in
// the kernel arguments, indexed by a head number known only at run time, is
// read through the memory hierarchy, one dependent round trip per access, in
// front of the first K/V or statistics load.
struct HeadMap {
    uint64_t str_mask;
    int32_t pool_heads;
    int32_t by_rank;              // 1: the pool holds the retrieval heads only
};
__host__ __device__ __forceinline__ bool head_streaming(const HeadMap &m, int kv) {
    return (m.str_mask >> kv) & 1u;
}
// rank of KV head kv among the streaming heads below it
__host__ __device__ __forceinline__ int streaming_rank(const HeadMap &m, int kv) {
    return __builtin_popcountll(m.str_mask & ((1ull << kv) - 1ull));
}
__host__ __device__ __forceinline__ int pool_slot(const HeadMap &m, int kv) {
    return m.by_rank ? kv - streaming_rank(m, kv) : kv;
}
// the KV head of the r-th retrieval head (r below the number of retrieval heads)
__host__ __device__ __forceinline__ int retrieval_head(const HeadMap &m, int r) {
    uint64_t z = ~m.str_mask;
    for (int i = 0; i < r; ++i) z &= z - 1ull;
    return __builtin_ctzll(z);
}

struct StatsArgs {
    const void *k;
    const uint16_t *k_sz;
    void *stats;
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *first_token;   // may be null
    int32_t batch, max_pages, num_kv_heads, head_dim, page_size, logical_page;
    int32_t n_heads_sel;          // number of KV heads processed
    int32_t lp_per_seq;           // logical pages covered per (sequence, head)
    int32_t dtype;
    uint8_t heads_sel[kMaxKvHeads];
    HeadMap hm;
};

struct ScoreArgs {
    const void *q;
    const void *stats;
    const void *k;                // the key pool: the current logical page is scored from its keys
    const uint16_t *k_sz;
    const int32_t *page_table;
    const int32_t *seq_lens;
    double *phys;                 // [B][H_kv][max_pages]
    int32_t batch, max_pages, num_q_heads, num_kv_heads, head_dim, page_size, logical_page;
    int32_t q_dtype, kv_dtype;
    int32_t aggregation;          // LSA_AGG_SUM | LSA_AGG_MAX
    int32_t n_ret;                // number of retrieval heads
    int32_t pages_per_block;      // physical pages per workgroup
    int32_t blocks_per_head;      // workgroups per (sequence, retrieval head)
    // fused top-K: the last score workgroup of a (sequence, head) selects its
    // pages; arrival counters [B][H_kv] head the workspace.  fused_pt is the
    // top-K's pages per thread (4, 8 or 16), 0 for a separate top-K launch.
    int32_t *counters;
    int32_t *selected;            // [B][H_kv][K]
    int32_t k_pages;              // K
    int32_t fused_pt;
    HeadMap hm;                   // retrieval head r of the workgroups: retrieval_head(hm, r)
    // the newest token's key rows [B][H_kv][D] (int4: D/2 bytes), or null: the
    // current logical page's last row (token t) is then read from the pool.
    // int4: k_new_sz [B][H_kv][2] holds t's page (s, z), used in place of the
    // pool's entry
    const void *k_new;
    const uint16_t *k_new_sz;
};

struct TopkArgs {
    const double *phys;
    const int32_t *seq_lens;
    int32_t *selected;            // [B][H_kv][K]
    int32_t batch, max_pages, num_kv_heads, page_size, k;
    int32_t n_ret;
    HeadMap hm;
};

struct DecodeArgs {
    const void *q;
    void *out;
    const void *k;
    const void *v;
    const uint16_t *k_sz;
    const uint16_t *v_sz;
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *selected;
    float *part;                  // partial records
    int32_t *counters;            // [B][H_kv] arrivals per (sequence, KV head); zero between calls
    void *stats;                  // may be null: refresh the current logical page's statistics
    int32_t batch, max_pages, num_q_heads, num_kv_heads, group, head_dim, page_size, logical_page;
    int32_t sel_k;                // K (row length of selected)
    int32_t sink, local;
    int32_t chunk_pages;              // pages per chunk (at most the kernel's decode_chunk_pages)
    int32_t chunks_ret, chunks_str;   // workgroups per (sequence, head) by kind
    int32_t chunks_max;               // record slots per (sequence, head)
    int32_t chunks_per_seq;           // workgroups per sequence
    float scale_log2;                 // softmax scale * log2(e)
    HeadMap hm;
    // streaming heads in a stream cache (sc_k == null: they are in the pool):
    // page m of (b, s = streaming_rank(hm, kv)) is cache page
    // (b * n_str + s) * (sink + ring) + (m < sink ? m : sink + (m - sink) % ring)
    const void *sc_k;
    const void *sc_v;
    const uint16_t *sc_k_sz;
    const uint16_t *sc_v_sz;
    int32_t sc_sink, sc_ring, n_str;
    // fused append (k_new != null): the newest token's K / V rows [B][H_kv][D]
    // (int4: [B][H_kv][D/2] codes and the page's (s, z) rows [B][H_kv][2]).  The
    // wavefront that reads the page of token t takes the token from these rows
    // and writes it to its page (pool or cache); for retrieval heads it also
    // updates the statistics of t's logical page (stats)
    const void *k_new;
    const void *v_new;
    const uint16_t *k_new_sz;
    const uint16_t *v_new_sz;
};

// The cache page of sequence page m of (b, s) in a stream cache.
__host__ __device__ __forceinline__ int64_t stream_cache_page(int b, int s, int m, int n_str, int sink, int ring) {
    return ((int64_t)b * n_str + s) * (sink + ring) + (m < sink ? m : sink + (m - sink) % ring);
}

struct AppendArgs {
    const void *k_new, *v_new;        // [B][H_kv][D] (int4: [B][H_kv][D/2] bytes)
    const uint16_t *k_new_sz, *v_new_sz;   // int4: [B][H_kv][2]
    void *k, *v;                      // pool
    uint16_t *k_sz, *v_sz;
    void *stats;                      // may be null
    const int32_t *page_table;
    const int32_t *seq_lens;
    int32_t batch, max_pages, num_kv_heads, head_dim, page_size, logical_page, dtype;
    HeadMap hm;
    void *sc_k, *sc_v;                // stream cache (null: streaming heads are in the pool)
    uint16_t *sc_k_sz, *sc_v_sz;
    int32_t sc_sink, sc_ring, n_str;
};

struct FillArgs {
    const void *k, *v;                // source pool, every KV head
    const uint16_t *k_sz, *v_sz;
    const int32_t *page_table;
    const int32_t *seq_lens;
    void *sc_k, *sc_v;
    uint16_t *sc_k_sz, *sc_v_sz;
    int32_t batch, max_pages, num_kv_heads, head_dim, page_size, dtype;
    int32_t sc_sink, sc_ring, n_str;
    uint8_t str_heads[kMaxKvHeads];   // the KV head of streaming slot s
};

struct PrefillArgs {
    const void *q;
    void *out;
    const void *k;
    const void *v;
    const int32_t *page_table;
    unsigned long long *tile_counter;
    int32_t seq_len, num_q_heads, num_kv_heads, group, head_dim, page_size;
    int32_t sink_blocks, local_blocks;
    int32_t n_qblocks;
    int32_t n_items;              // work items (kv head, query tile group, head group)
    int32_t head_groups;          // query-head groups of 4 per KV head
    int32_t q_tiles;              // query tiles per work item (4 / G when G < 4, else 1)
    int32_t n_qgroups;            // ceil(n_qblocks / q_tiles)
    float scale_log2;
    int32_t n_ret, n_str;         // retrieval / streaming KV heads
    uint8_t ret_heads[kMaxKvHeads];
    uint8_t str_heads[kMaxKvHeads];
    // static block mask (CSR): per KV head, row_ptr[h * (n_qblocks + 1) + a]
    // .. [.. + a + 1] index col_idx, the key tiles of query tile a
    const int32_t *row_ptr;
    const int32_t *col_idx;
    int32_t nnz;
    // optional work order of a static mask: order[blockIdx] = (kv * n_qblocks + a) * head_groups + hg
    const int32_t *order;
};

// ----------------------------------------------------------------------------
// launchers (each returns hipSuccess or the launch error)
// ----------------------------------------------------------------------------

hipError_t launch_stats(const StatsArgs &a, hipStream_t s);
hipError_t launch_score(const ScoreArgs &a, hipStream_t s);
int score_pages_per_block(int kv_dtype, int head_dim, int page_size, int logical_page, int fused_pt, bool agg_max);
int score_loop_pages_per_block(int batch, int n_ret, int max_pages, int page_size, int logical_page, int kv_dtype);
int topk_max_pages();
int score_fused_pt(int max_pages, bool agg_max);   // top-K pages per thread inside the score kernel, 0: a separate launch
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int q_dtype, int kv_dtype, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t s);
hipError_t launch_append(const AppendArgs &a, hipStream_t s);
hipError_t launch_stream_fill(const FillArgs &a, hipStream_t s);

}  // namespace lsa
