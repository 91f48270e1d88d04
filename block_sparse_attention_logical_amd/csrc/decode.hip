// Block-sparse paged decode attention for retrieval and streaming heads
// (LServe explainer, 技術的詳細 / 静的スパーシティ: streaming heads see the sink
// and the recent tokens; 動的スパーシティ and the figure: retrieval heads read
// only their top-K physical pages; 統一ブロックスパースアテンション: one
// block-sparse kernel serves both head kinds; abstract page: a constant number
// of KV pages per step; the KV4 co-design pairs the sparse path with 4-bit KV).
//
// Work decomposition (split-KV).  The attended page list of a (sequence, KV
// head) is cut into chunks; one workgroup takes a chunk (wavefront 0 resolves
// the chunk's pool pages into LDS), each wavefront streams its share with an
// online softmax, the wavefronts' states are merged in LDS and one partial
// record (max, sum, unnormalised output) is written per chunk.  The MFMA path
// runs four wavefronts of up to 128 tokens each (up to eight pages of 64
// tokens per chunk); the f32 path four wavefronts of one page.  The last workgroup of a
// (sequence, KV head) to finish merges every record in chunk order (so the
// result does not depend on arrival order) and writes the output.  The
// hand-off avoids a device-scope fence (an L2 writeback on this part): the
// records are written and read with agent-scope stores and loads, which go to
// the coherence point past the per-XCD L2s, and a workgroup counts its arrival
// only after its record stores have completed (s_waitcnt vmcnt(0)).  The
// arrival counter is an agent-scope atomic; the last arrival resets it to
// zero.  Every K/V page read serves all G query heads.
//
// MFMA path (bf16 and int4 pools).  Both contractions run on
// v_mfma_f32_16x16x32_bf16 straight from registers.  QK^T is computed
// transposed (tokens in M, heads in N) as two 16-token tiles per 32-token
// block; with the pool's key tiles every channel step of a tile is one
// contiguous 1 KiB read.  A lane's scores (4 tokens of each tile) are
// regrouped with two permlane swaps into 8 consecutive tokens of one head, the
// B operand of PV; the A operand of PV (one channel, 8 consecutive tokens of
// the value rows) is again a contiguous read.  Heads occupy the N dimension,
// padded to 16 with zero queries.  A wavefront walks its 32-token blocks
// through a ring of register buffers: the loads of the next blocks (one more
// for bf16, three more for int4) are in flight while a block is computed, so
// the wavefront's memory stream never drains between blocks.  Every slot of
// the ring is always loaded (a block that needs no keys re-reads the
// wavefront's first needed block, which is already on its way to the caches),
// so the wait before each block counts exactly the loads issued after it.
// The block loads carry the non-temporal hint: each K/V byte is read once per
// launch, and the stream should not displace the lines the launch reuses.
//
// int4 pools.  A code c (0..15) becomes the bf16 bit pattern 0x4300 | c, which
// is exactly 128 + c, so the MFMAs see exact operands; the offset and the
// page's zero point come off afterwards: q.k = s_k (q.(128 + c) - (128 + z_k)
// sum(q)), and for values the probabilities are pre-multiplied by s_v and the
// per-head term (128 + z_v) * sum(p') is subtracted at the end, with p' the
// very bf16 weights fed to the MFMA so the offset cancels exactly.
#include "lsa_internal.h"

namespace lsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

struct WorkItem {
    int b, kv, chunk, t, L;
    int t_pool;          // the last token read from memory: t, or t - 1 when this launch appends t
    bool streaming;
};

__device__ __forceinline__ WorkItem decode_item(const DecodeArgs &a) {
    WorkItem w;
    w.b = blockIdx.x / a.chunks_per_seq;
    int off = blockIdx.x % a.chunks_per_seq;
    int kv = 0;
    for (; kv < a.num_kv_heads; ++kv) {
        const int c = head_streaming(a.hm, kv) ? a.chunks_str : a.chunks_ret;
        if (off < c) break;
        off -= c;
    }
    w.kv = kv;
    w.chunk = off;
    w.streaming = head_streaming(a.hm, kv);
    return w;
}

// Slots of the per-workgroup page list in LDS: t, L, then the sequence pages
// of the chunk, then their pool pages (-1: no page).
constexpr int kListSlots = 2 + 2 * kMaxChunkPages;

// Wavefront 0 of a workgroup resolves the pages of its chunk into CP list
// slots: the attended pages of a (sequence, KV head) in ascending order are
// the selection row (valid entries first, then -1) followed by the current
// page when the row lacks it (retrieval heads), or the sink pages followed by
// the local window (streaming heads); with c = chunk_pages the chunk takes
// list entries c * chunk .. c * chunk + c - 1 into slots 0 .. c - 1, the other
// slots hold no page.  seq_lens and the selection entries are loaded
// together, then the page-table entries: two dependent loads in all.
template <int CP>
__device__ __forceinline__ void wg_pages(const DecodeArgs &a, const WorkItem &w, int *list) {
    static_assert(CP <= kMaxChunkPages && (CP & (CP - 1)) == 0, "chunk pages");
    const int lane = threadIdx.x % kWave;
    const int NP = a.page_size;
    const bool slot_used = lane < a.chunk_pages;
    const int i = w.chunk * a.chunk_pages + lane;      // list index of this lane's page (lanes < chunk_pages)
    const int32_t *sel = w.streaming ? nullptr : a.selected + ((size_t)w.b * a.num_kv_heads + w.kv) * a.sel_k;
    int m_row = -1, m_i = -1;
    if (sel) {
        if (lane < a.sel_k) m_row = sel[lane];
        if (slot_used && i < a.sel_k) m_i = sel[i];
    }
    const int L = a.seq_lens[w.b];
    const int t = L - 1, cur = t / NP;
    int page = -1;
    if (w.streaming) {
        const int sink_end = min(a.sink, t + 1);          // tokens [0, sink_end)
        const int n_sink = (sink_end + NP - 1) / NP;
        const int local_first = max(max(0, t - a.local + 1) / NP, n_sink);
        const int n = n_sink + max(0, cur - local_first + 1);
        if (slot_used && i < n) page = i < n_sink ? i : local_first + (i - n_sink);
    } else {
        int cnt = __popcll(__ballot(m_row >= 0));
        bool in = __ballot(m_row == cur) != 0;
        for (int j0 = kWave; j0 < a.sel_k; j0 += kWave) {
            const int m = j0 + lane < a.sel_k ? sel[j0 + lane] : -1;
            cnt += __popcll(__ballot(m >= 0));
            in |= __ballot(m == cur) != 0;
        }
        const int n = cnt + (in ? 0 : 1);
        if (slot_used && i < n) page = i < cnt ? m_i : cur;
    }
    int pool = -1;                    // pool page, or the stream-cache page of a streaming head
    if (lane < CP && page >= 0)
        pool = w.streaming && a.sc_k
                   ? (int)stream_cache_page(w.b, streaming_rank(a.hm, w.kv), page, a.n_str, a.sc_sink, a.sc_ring)
                   : a.page_table[(size_t)w.b * a.max_pages + page];
    if (lane == 0) { list[0] = t; list[1] = L; }
    if (lane < CP) { list[2 + lane] = page; list[2 + CP + lane] = pool; }
}

// Is token p attended and read from memory (p <= t_pool)?
__device__ __forceinline__ bool token_visible(const DecodeArgs &a, const WorkItem &w, int p) {
    // bitwise, not short-circuit: no branch inside the block compute
    return (p <= w.t_pool) & (!w.streaming | (p < a.sink) | ((w.t - p) < a.local));
}

// Does the run of n tokens starting at tok0 hold any attended token read from memory?
__device__ __forceinline__ bool block_needed(const DecodeArgs &a, const WorkItem &w, int tok0, int n) {
    if (tok0 > w.t_pool) return false;
    if (!w.streaming) return true;
    const int p_last = min(tok0 + n - 1, w.t_pool);
    return tok0 < a.sink || (w.t - p_last) < a.local;
}

// Recompute the statistics of the logical page that holds token t (retrieval
// heads keep them for later selections).  One wavefront; lanes own channels.
__device__ __forceinline__ void refresh_current_stats(const DecodeArgs &a, const WorkItem &w, int kv_dtype) {
    const int lane = threadIdx.x % kWave;
    const int NL = a.logical_page, NP = a.page_size, D = a.head_dim;
    const int g = NP / NL;
    const int j = w.t / NL;
    const int m = j / g, jl = j % g;
    const int row0 = jl * NL, rows = w.t - j * NL + 1;
    const int pool = a.page_table[(size_t)w.b * a.max_pages + m];
    const size_t hp = (size_t)pool * a.hm.pool_heads + pool_slot(a.hm, w.kv);
    const size_t page_base = hp * NP * D;
    if (kv_dtype == LSA_INT4) {
        if (lane >= D / 2) return;
        const uint8_t *k = static_cast<const uint8_t *>(a.k);
        uint32_t lo_min = 15, lo_max = 0, hi_min = 15, hi_max = 0;
        for (int r = 0; r < rows; ++r) {
            const uint32_t byte = k[(page_base + key_offset(row0 + r, 2 * lane, D, block_shift(NP))) / 2];
            lo_min = min(lo_min, byte & 15u); lo_max = max(lo_max, byte & 15u);
            hi_min = min(hi_min, byte >> 4); hi_max = max(hi_max, byte >> 4);
        }
        uint8_t *st = static_cast<uint8_t *>(a.stats) + (hp * g + jl) * D + 2 * lane;
        *reinterpret_cast<uint16_t *>(st) = uint16_t((lo_min | (lo_max << 4)) | ((hi_min | (hi_max << 4)) << 8));
        return;
    }
    const int cpl = D / 64;
    for (int c = 0; c < cpl; ++c) {
        const int ch = lane * cpl + c;
        float mn = __builtin_inff(), mx = -__builtin_inff();
        for (int r = 0; r < rows; ++r) {
            float x;
            const size_t off = page_base + key_offset(row0 + r, ch, D, block_shift(NP));
            if (kv_dtype == LSA_BF16)
                x = bf16_to_f32(static_cast<const uint16_t *>(a.k)[off]);
            else
                x = static_cast<const float *>(a.k)[off];
            mn = fminf(mn, x);
            mx = fmaxf(mx, x);
        }
        const size_t base = ((hp * g + jl) * 2) * D + ch;
        if (kv_dtype == LSA_BF16) {
            static_cast<uint16_t *>(a.stats)[base] = uint16_t(__float_as_uint(mn) >> 16);
            static_cast<uint16_t *>(a.stats)[base + D] = uint16_t(__float_as_uint(mx) >> 16);
        } else {
            static_cast<float *>(a.stats)[base] = mn;
            static_cast<float *>(a.stats)[base + D] = mx;
        }
    }
}

// The value itself, hidden from the optimiser: the query's channels are
// converted to fp32 once for the int4 query sum before the key loop and again
// for the appended token's logit after it; without this the first conversions
// would be kept live across the whole loop to serve the second.
__device__ __forceinline__ uint4 opaque(uint4 v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
    return v;
}

// Fused append: write token t (its K / V rows staged in LDS) into its page
// and, for retrieval heads, fold it into the statistics of its logical page
// (a logical page the token opens starts from it; otherwise min / max take it
// in, exactly).  Lanes own channels; an int4 value byte also holds the
// neighbouring token's code, which is kept.
template <int KVT, int D, int NP, int PPW>
__device__ __forceinline__ void append_write(const DecodeArgs &a, const WorkItem &w, int j_new, const size_t (&hp)[PPW],
                                             const int (&pg)[PPW], const void *kpool, const void *vpool,
                                             const uint16_t *kszp, const uint16_t *vszp, uint32_t ksz_n,
                                             uint32_t vsz_n, const uint8_t *row8, int lane) {
    (void)pg;
    constexpr int BS = block_shift(NP);
    constexpr int ROW = KVT == LSA_INT4 ? D / 2 : 2 * D;     // bytes of the staged K row (then the V row)
    size_t hpn = 0;                                          // hp[j_new], without a dynamic register index
#pragma unroll
    for (int j = 0; j < PPW; ++j) hpn = j == j_new ? hp[j] : hpn;
    const size_t base = hpn * NP * D;
    const int slot = w.t % NP, NL = a.logical_page, g = NP / NL, jl = slot / NL;
    const bool opens = slot % NL == 0;
    const bool upd = a.stats != nullptr && !w.streaming;
    if constexpr (KVT == LSA_INT4) {
        uint8_t *k8 = const_cast<uint8_t *>(static_cast<const uint8_t *>(kpool));
        uint8_t *v8 = const_cast<uint8_t *>(static_cast<const uint8_t *>(vpool));
        for (int i = lane; i < D / 2; i += kWave)             // key byte i: channels 2i, 2i + 1
            k8[(base + key_offset(slot, 2 * i, D, BS)) / 2] = row8[i];
        for (int c = lane; c < D; c += kWave) {
            const uint32_t code = (row8[ROW + c / 2] >> (4 * (c & 1))) & 15u;
            uint8_t *vb = v8 + (base + value_offset(slot, c, D, BS)) / 2;
            const uint32_t old = *vb;
            *vb = (uint8_t)((slot & 1) ? ((old & 0x0Fu) | (code << 4)) : ((old & 0xF0u) | code));
            if (upd) {
                const uint32_t kc = (row8[c / 2] >> (4 * (c & 1))) & 15u;
                uint8_t *st = static_cast<uint8_t *>(a.stats) + (hpn * g + jl) * D + c;
                const uint32_t ob = opens ? 0u : *st;
                *st = (uint8_t)(opens ? (kc | (kc << 4)) : (min(ob & 15u, kc) | (max(ob >> 4, kc) << 4)));
            }
        }
        if (lane == 0) {
            *reinterpret_cast<uint32_t *>(const_cast<uint16_t *>(kszp) + hpn * 2) = ksz_n;
            *reinterpret_cast<uint32_t *>(const_cast<uint16_t *>(vszp) + hpn * 2) = vsz_n;
        }
    } else {
        uint16_t *kd = const_cast<uint16_t *>(static_cast<const uint16_t *>(kpool)) + base;
        uint16_t *vd = const_cast<uint16_t *>(static_cast<const uint16_t *>(vpool)) + base;
        const uint16_t *kr = reinterpret_cast<const uint16_t *>(row8);
        const uint16_t *vr = reinterpret_cast<const uint16_t *>(row8 + ROW);
        uint16_t *st = static_cast<uint16_t *>(a.stats) + ((hpn * g + jl) * 2) * D;
        for (int c = lane; c < D; c += kWave) {
            kd[key_offset(slot, c, D, BS)] = kr[c];
            vd[value_offset(slot, c, D, BS)] = vr[c];
            if (upd) {
                const float x = bf16_to_f32(kr[c]);
                const float mn = opens ? x : fminf(bf16_to_f32(st[c]), x);
                const float mx = opens ? x : fmaxf(bf16_to_f32(st[D + c]), x);
                st[c] = uint16_t(__float_as_uint(mn) >> 16);          // exact: bf16 values
                st[D + c] = uint16_t(__float_as_uint(mx) >> 16);
            }
        }
    }
}

__device__ __forceinline__ void store_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent2(float *p, float x, float y) {
    const unsigned long long u = (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent2(const float *p) {
    const unsigned long long u =
        __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float(uint32_t(u)), __uint_as_float(uint32_t(u >> 32)));
}

// Merge the softmax states of the NW wavefronts held in LDS and write this
// chunk's record (m[16], l[16], o[G][D]) with agent-scope stores.  LDS layout
// per wave: m[16], l[16], o[16][D].
// With `extra`, a one-token state follows the NW wavefront states: a logit
// per head (16 floats) and the token's value row (D floats), weight 1; its
// logit is -inf in workgroups that do not hold the token.
template <int NW>
__device__ __forceinline__ void merge_waves_and_store(const DecodeArgs &a, const WorkItem &w,
                                                      const float *lds, int D, bool extra) {
    const int G = a.group;
    const int wave_stride = 32 + 16 * D;
    const size_t rec_size = 32 + (size_t)G * D;
    const float *nt = lds + NW * wave_stride;
    float *rec = a.part + (((size_t)w.b * a.num_kv_heads + w.kv) * a.chunks_max + w.chunk) * rec_size;
    for (int pi = threadIdx.x; pi < G * D / 2; pi += blockDim.x) {
        const int h = (2 * pi) / D, d = 2 * pi - h * D;
        float M = -__builtin_inff();
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, lds[wv * wave_stride + h]);
        const float mt = extra ? nt[h] : -__builtin_inff();
        M = fmaxf(M, mt);
        float acc0 = 0.f, acc1 = 0.f, lsum = 0.f;
        if (M != -__builtin_inff()) {
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                const float mw = lds[wv * wave_stride + h];
                const float wt = mw == -__builtin_inff() ? 0.f : exp2_fast(mw - M);
                acc0 += wt * lds[wv * wave_stride + 32 + h * D + d];
                acc1 += wt * lds[wv * wave_stride + 32 + h * D + d + 1];
                lsum += wt * lds[wv * wave_stride + 16 + h];
            }
            if (mt != -__builtin_inff()) {
                const float wt = exp2_fast(mt - M);
                acc0 += wt * nt[16 + d];
                acc1 += wt * nt[16 + d + 1];
                lsum += wt;
            }
        }
        store_agent2(rec + 32 + 2 * pi, acc0, acc1);
        if (d == 0) {
            store_agent(rec + h, M);
            store_agent(rec + 16 + h, lsum);
        }
    }
}

// Count this chunk's arrival; the last workgroup of the (sequence, KV head)
// merges the records of all its chunks, in chunk order, into out, loading CB
// chunks' records per memory round trip.
template <typename OutT, int CB>
__device__ __forceinline__ void finish_head(const DecodeArgs &a, const WorkItem &w, int D) {
    __shared__ int s_last;
    // this wavefront's record stores have reached the coherence point
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int nchunks = w.streaming ? a.chunks_str : a.chunks_ret;
    if (threadIdx.x == 0) {
        int32_t *cnt = a.counters + (size_t)w.b * a.num_kv_heads + w.kv;
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == nchunks - 1;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;

    // a thread merges four channels
    const int G = a.group;
    const size_t rec_size = 32 + (size_t)G * D;
    const float *rec0 = a.part + ((size_t)w.b * a.num_kv_heads + w.kv) * a.chunks_max * rec_size;
    for (int qi = threadIdx.x; qi < G * D / 4; qi += blockDim.x) {
        const int hh = (4 * qi) / D, d = 4 * qi - hh * D;
        float M = -__builtin_inff(), L = 0.f;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < nchunks; c0 += CB) {
            float mv[CB], lv[CB];
            float2 ov[CB][2];
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const float *rec = rec0 + (size_t)(c0 + c) * rec_size;
                const bool in = c0 + c < nchunks;
                mv[c] = in ? load_agent(rec + hh) : -__builtin_inff();
                lv[c] = in ? load_agent(rec + 16 + hh) : 0.f;
                ov[c][0] = in ? load_agent2(rec + 32 + 4 * qi) : make_float2(0.f, 0.f);
                ov[c][1] = in ? load_agent2(rec + 32 + 4 * qi + 2) : make_float2(0.f, 0.f);
            }
            float Mb = M;
#pragma unroll
            for (int c = 0; c < CB; ++c) Mb = fmaxf(Mb, mv[c]);
            const float sc = M == -__builtin_inff() ? 0.f : exp2_fast(M - Mb);
            L *= sc;
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] *= sc;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const float e = mv[c] == -__builtin_inff() ? 0.f : exp2_fast(mv[c] - Mb);
                L += e * lv[c];
                acc[0] += e * ov[c][0].x;
                acc[1] += e * ov[c][0].y;
                acc[2] += e * ov[c][1].x;
                acc[3] += e * ov[c][1].y;
            }
            M = Mb;
        }
        const size_t o = ((size_t)w.b * a.num_q_heads + (size_t)w.kv * G + hh) * D + d;
        if constexpr (sizeof(OutT) == 2) {
            uint2 pk;
            pk.x = uint32_t(f32_to_bf16_rne(acc[0] / L)) | (uint32_t(f32_to_bf16_rne(acc[1] / L)) << 16);
            pk.y = uint32_t(f32_to_bf16_rne(acc[2] / L)) | (uint32_t(f32_to_bf16_rne(acc[3] / L)) << 16);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + o) = pk;
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + o) =
                make_float4(acc[0] / L, acc[1] / L, acc[2] / L, acc[3] / L);
        }
    }
}

// The eight codes of `w` (byte k: code 2k in its low nibble, code 2k + 1 in
// its high nibble) as bf16 bit patterns 0x4300 | c (= 128 + c), in the order
// c0 c2 c4 c6 c1 c3 c5 c7.  The low and the high nibbles are masked out once;
// one byte permute per dword then interleaves two of them with the exponent
// byte 0x43 of a constant operand (v_perm_b32 selector bytes 0..3 pick bytes
// of the second operand, 4..7 bytes of the first).  The operand that meets
// these in the MFMA k dimension is stored in the same order.
__device__ __forceinline__ uint4 nibbles_bf16x8_split(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    constexpr uint32_t E = 0x43434343u;
    return make_uint4(__builtin_amdgcn_perm(E, lo, 0x04010400u), __builtin_amdgcn_perm(E, lo, 0x04030402u),
                      __builtin_amdgcn_perm(E, hi, 0x04010400u), __builtin_amdgcn_perm(E, hi, 0x04030402u));
}

// Eight bf16 values (x0 .. x7, two to a dword) reordered to x0 x2 x4 x6 x1 x3
// x5 x7, the order of nibbles_bf16x8_split.
__device__ __forceinline__ uint4 split_order(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
    return make_uint4(__builtin_amdgcn_perm(d1, d0, 0x05040100u), __builtin_amdgcn_perm(d3, d2, 0x05040100u),
                      __builtin_amdgcn_perm(d1, d0, 0x07060302u), __builtin_amdgcn_perm(d3, d2, 0x07060302u));
}

__device__ __forceinline__ uint32_t pick(const uint4 &u, int i) {
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// ---------------------------------------------------------------------------
// MFMA kernel, bf16 or int4 pool, bf16 q
// ---------------------------------------------------------------------------
template <int D, int KVT, int NP>
__global__ __launch_bounds__(kDecodeWaves * kWave, decode_waves_per_simd(KVT, NP)) void decode_mfma_kernel(DecodeArgs a) {
    constexpr bool I4 = KVT == LSA_INT4;
    // 16-token pages: a 32-token block is two pages, QK^T tile T (and the
    // value rows of lanes with g4 / 2 == T) coming from page 2i + T of block i
    constexpr bool HALF = NP == 16;
    constexpr int BS = block_shift(NP);   // log2 of the tokens per layout block
    constexpr int NS = D / 32;            // MFMA k-steps over channels
    constexpr int NDT = D / 16;           // output channel tiles
    constexpr int NB = HALF ? 1 : NP / 32;   // 32-token blocks per page
    constexpr int PPW = decode_pages_per_wave(KVT, NP);
    constexpr int NBW = HALF ? PPW / 2 : PPW * NB;   // 32-token blocks per wavefront
    constexpr int CP = kDecodeWaves * PPW;
    constexpr int BIF = I4 ? (NBW < 4 ? NBW : 4) : 2;   // blocks in flight (ring size)
    extern __shared__ float lds[];
    WorkItem w = decode_item(a);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int h = lane & 15, g4 = lane >> 4;
    const int G = a.group;

    // B operand of QK^T: column h = query head.  bf16 pools: step s holds
    // channels 32s + 8*g4 + j; int4 pools: channels (D/4)*g4 + 8s + j (so that a
    // lane's steps cover one contiguous run of codes of its key row), stored
    // in the order j = 0 2 4 6 1 3 5 7 of the unpacked codes.
    bf16x8 qb[NS];
    float qsum = 0.f;                      // int4: sum over channels of q_h
    {
        const uint16_t *q = static_cast<const uint16_t *>(a.q) +
                            ((size_t)w.b * a.num_q_heads + (size_t)w.kv * G + min(h, G - 1)) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            uint4 raw = *reinterpret_cast<const uint4 *>(q + (I4 ? (D / 4) * g4 + 8 * s : 32 * s + 8 * g4));
            if (h >= G) raw = make_uint4(0, 0, 0, 0);
            if constexpr (I4) {
#pragma unroll
                for (int e = 0; e < 4; ++e) qsum += bf16_lo(pick(raw, e)) + bf16_hi(pick(raw, e));
                raw = split_order(raw.x, raw.y, raw.z, raw.w);     // the order of the unpacked codes
            }
            qb[s] = __builtin_bit_cast(bf16x8, raw);
        }
        if constexpr (I4) {
            qsum = sum_xor32(sum_xor16(qsum));
        }
    }
    __shared__ int s_list[kListSlots];
    // fused append: the token's K row, V row and (int4) its (s, z) pairs
    constexpr int kNewRow = I4 ? D / 2 : 2 * D;       // bytes of one row
    __shared__ uint4 s_new[2 * kNewRow / 16 + 1];
    if (wave == 0) wg_pages<CP>(a, w, s_list);
    if (wave == 2 && a.k_new && lane < 16) lds[kDecodeWaves * (32 + 16 * D) + lane] = -__builtin_inff();
    if (wave == 1 && a.k_new) {
        const size_t row = ((size_t)w.b * a.num_kv_heads + w.kv) * kNewRow;
        if (lane < kNewRow / 16) {
            s_new[lane] = *reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(a.k_new) + row + 16 * lane);
            s_new[kNewRow / 16 + lane] =
                *reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(a.v_new) + row + 16 * lane);
        }
        if (I4 && lane == 0) {
            const size_t i2 = ((size_t)w.b * a.num_kv_heads + w.kv) * 2;
            s_new[2 * kNewRow / 16] = make_uint4(*reinterpret_cast<const uint32_t *>(a.k_new_sz + i2),
                                                 *reinterpret_cast<const uint32_t *>(a.v_new_sz + i2), 0u, 0u);
        }
    }
    __syncthreads();
    w.t = __builtin_amdgcn_readfirstlane(s_list[0]);
    w.L = __builtin_amdgcn_readfirstlane(s_list[1]);
    w.t_pool = a.k_new ? w.t - 1 : w.t;

    // this wavefront's pages: chunk slots PPW*wave .. PPW*wave + PPW - 1, as
    // (page, head) units of the pool, or pages of the stream cache
    const bool in_cache = w.streaming && a.sc_k != nullptr;
    const void *kpool = in_cache ? a.sc_k : a.k;
    const void *vpool = in_cache ? a.sc_v : a.v;
    const uint16_t *kszp = in_cache ? a.sc_k_sz : a.k_sz;
    const uint16_t *vszp = in_cache ? a.sc_v_sz : a.v_sz;
    const size_t hp_mul = in_cache ? 1 : (size_t)a.hm.pool_heads;
    const size_t hp_add = in_cache ? 0 : pool_slot(a.hm, w.kv);
    int pg[PPW];
    size_t hp[PPW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        pg[j] = __builtin_amdgcn_readfirstlane(s_list[2 + PPW * wave + j]);
        const int pool = __builtin_amdgcn_readfirstlane(s_list[2 + CP + PPW * wave + j]);
        hp[j] = (size_t)max(pool, 0) * hp_mul + hp_add;
    }
    // block i of the wavefront: page slot i / NB, 32-token block i % NB of that
    // page; with 16-token pages, tile T of block i is page slot 2i + T.  Per
    // (block, tile), as bits of scalar registers (wavefront-uniform; arrays of
    // flags and positions cost a scalar register or a pair each, and the
    // instances with many blocks per wavefront ran out of them): need (bit
    // 2i + T) whether it holds an attended token, full (bit i) whether all 32
    // tokens of the block are attended and read from memory (its scores and
    // values then need no masking).  A tile's first token position is
    // recomputed from the page slot where it is used.
    auto slot_of = [&](int i, int T) { return HALF ? 2 * i + T : i / NB; };
    auto tok_of = [&](int i, int T) { return HALF ? pg[2 * i + T] * NP : pg[i / NB] * NP + 32 * (i % NB) + 16 * T; };
    uint32_t need_bits = 0, full_bits = 0;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        bool nd[2];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            if constexpr (HALF) nd[T] = pg[2 * i + T] >= 0 && block_needed(a, w, tok_of(i, T), NP);
            else nd[T] = pg[i / NB] >= 0 && block_needed(a, w, tok_of(i, 0), 32);
        }
        bool f = nd[0] & nd[1];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const int p0 = tok_of(i, T), p1 = p0 + 15;
            f &= (p1 <= w.t_pool) & (!w.streaming | (p1 < a.sink) | (w.t - p0 < a.local));
        }
        need_bits |= (nd[0] ? 1u : 0u) << (2 * i);
        need_bits |= (nd[1] ? 1u : 0u) << (2 * i + 1);
        full_bits |= (f ? 1u : 0u) << i;
    }
    need_bits = __builtin_amdgcn_readfirstlane(need_bits);
    full_bits = __builtin_amdgcn_readfirstlane(full_bits);
    auto need_t = [&](int i, int T) -> bool { return (need_bits >> (2 * i + T)) & 1u; };
    const bool any = need_bits != 0;

    floatx4 o[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff(), l_run = 0.f;
    float corr = 0.f;                      // int4: (128 + z_v) * sum of fed weights (per lane)

    // fused append: the page slot of token t in this wavefront (-1: none;
    // wavefront-uniform).  The ring reads tokens up to t - 1; this wavefront
    // adds token t from the staged rows after the ring and writes it out.
    int j_new = -1;
    if (a.k_new) {
#pragma unroll
        for (int j = 0; j < PPW; ++j) j_new = pg[j] == w.t / NP ? j : j_new;
    }
    // the token's K and V rows and (int4) its page's scale and zero point,
    // staged in LDS by wavefront 1 while wavefront 0 resolved the page list
    const uint8_t *s_new8 = reinterpret_cast<const uint8_t *>(s_new);
    uint32_t ksz_n = 0, vsz_n = 0;
    if (I4 && j_new >= 0) {               // (wavefront-uniform: scalar registers)
        ksz_n = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_new[2 * kNewRow / 16].x);
        vsz_n = (uint32_t)__builtin_amdgcn_readfirstlane((int)s_new[2 * kNewRow / 16].y);
    }

    // QK^T tile T of a 32-token block holds tokens 16T .. 16T + 15 on MFMA
    // rows (row rho = token 16T + rho, one contiguous 1 KiB key-tile read per
    // channel step); a lane's result registers hold tokens 16T + 4*g4 + r.
    const int rho = lane & 15;

    if (any) {
        float sk[PPW], zk[PPW], sv[PPW], zv[PPW];
#pragma unroll
        for (int j = 0; j < PPW; ++j) {
            sk[j] = 1.f; zk[j] = 0.f; sv[j] = 1.f; zv[j] = 0.f;
            if constexpr (I4) {
                if (pg[j] >= 0) {
                    // (the page of a token being appended may not have its pair in memory yet)
                    const uint32_t ksz = j == j_new ? ksz_n : *reinterpret_cast<const uint32_t *>(kszp + hp[j] * 2);
                    const uint32_t vsz = j == j_new ? vsz_n : *reinterpret_cast<const uint32_t *>(vszp + hp[j] * 2);
                    sk[j] = fp16_bits_to_f32(uint16_t(ksz)); zk[j] = fp16_bits_to_f32(uint16_t(ksz >> 16));
                    sv[j] = fp16_bits_to_f32(uint16_t(vsz)); zv[j] = fp16_bits_to_f32(uint16_t(vsz >> 16));
                }
            }
        }
        // source of each ring load: the block (tile) itself, or the first
        // needed tile (its page slot and its block within that page)
        size_t f_hp = 0;
        int f_kb = 0;
        {
            const int ft = __builtin_ctz(need_bits), fi = ft >> 1, fT = ft & 1;
#pragma unroll
            for (int j = 0; j < PPW; ++j)
                if (j == (HALF ? 2 * fi + fT : fi / NB)) f_hp = hp[j];
            f_kb = HALF ? 0 : fi % NB;
        }
        auto src_hp = [&](int i, int T) -> size_t { return need_t(i, T) ? hp[slot_of(i, T)] : f_hp; };
        auto src_kb = [&](int i) -> int { return ((need_bits >> (2 * i)) & 3u) ? (HALF ? 0 : i % NB) : f_kb; };

        uint4 kr[BIF][2][I4 ? 1 : NS];
        uint4 vr[BIF][I4 ? 1 : NDT];
        // int4 values.  The PV operand wants, per output tile dt, the 4 bytes
        // of tokens 8*g4 .. 8*g4+7 of channel 16*dt + h: one dword per tile,
        // which as loads of their own move 256 bytes per instruction, and
        // loads that narrow cap the stream far below the HBM rate.  So lane
        // (h, g4) loads whole 16-byte channel rows (all 32 tokens) instead,
        // those of tiles (NDT/4)*g4 + j, and a 4 x 4 transpose across the
        // four lane groups of h (permlane swaps) hands every lane its dwords.
        // 16-token pages keep per-tile dword loads (a lane's page depends on
        // its token group there).
        constexpr int VRW = I4 && !HALF ? NDT / 4 : 1;    // 16-byte value rows per lane and block
        uint4 vq[BIF][VRW];
        uint32_t vr4[BIF][I4 && HALF ? NDT : 1];
        // Ring loads go through a buffer resource over the page they read (its
        // base in scalar registers), with the lane's byte offset within a
        // block, the same for every block, formed here once; the block, tile,
        // channel-step and output-tile terms are wavefront-uniform scalar
        // offsets.  Every address is the page layout's own, as with plain
        // loads.  The value rows of 16-token pages (a lane's page depends on
        // its token group) stay plain loads.
        constexpr int kPageBytes = I4 ? NP * D / 2 : NP * D * 2;
        auto to_bytes = [](size_t elems) -> uint32_t { return (uint32_t)(I4 ? elems / 2 : elems * 2); };
        const uint32_t k_lane = to_bytes(key_offset(rho, I4 ? (D / 4) * g4 : 8 * g4, D, BS));
        const uint32_t v_lane = to_bytes(value_offset(8 * g4, h, D, BS));
        const uint32_t v_row_lane = to_bytes(value_offset(0, 16 * VRW * g4 + h, D, BS));   // int4 value rows
        // ---- issue every K and V load of block i into ring slot e
        auto issue = [&](int e, int i) __attribute__((always_inline)) {
            const int kb = src_kb(i);
            // the pages of tiles 0 and 1 (element offsets), and the block's and
            // the tiles' offsets within them: tile T holds tokens 16T .. 16T + 15
            // of block kb, or is page slot 2i + T (16-token pages)
            const size_t kbase[2] = {src_hp(i, 0) * NP * D, src_hp(i, 1) * NP * D};
            const uint32_t blk = HALF ? 0u : (uint32_t)(kb * 32 * D);
            auto tile_el = [&](int T) -> uint32_t { return HALF ? 0u : blk + 512u * T; };
            if constexpr (I4) {
                const uint8_t *k8 = static_cast<const uint8_t *>(kpool);
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    const uint8_t *page = k8 + kbase[T] / 2;
                    if constexpr (D == 128) {
                        kr[e][T][0] = buffer_stream16(page, kPageBytes, k_lane, to_bytes(tile_el(T)));
                    } else {
                        const uint2 u = buffer_stream8(page, kPageBytes, k_lane, to_bytes(tile_el(T)));
                        kr[e][T][0] = make_uint4(u.x, u.y, 0, 0);
                    }
                }
                const uint8_t *v8 = static_cast<const uint8_t *>(vpool);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    if constexpr (HALF) {
                        // tokens 8*(g4%2) .. of page 2i + g4/2
                        const size_t vbase = g4 < 2 ? kbase[0] : kbase[1];
                        vr4[e][dt] = load_stream4(v8 + (vbase + value_offset(8 * (g4 & 1), 16 * dt + h, D, BS)) / 2);
                    }
                }
                if constexpr (!HALF) {
                    // the row of channel 16 * (VRW * g4 + j) + h: 16 channels = 512 codes further per j
#pragma unroll
                    for (int j = 0; j < VRW; ++j)
                        vq[e][j] = buffer_stream16(v8 + kbase[0] / 2, kPageBytes, v_row_lane, to_bytes(blk + 512u * j));
                }
            } else {
                const uint16_t *kp = static_cast<const uint16_t *>(kpool);
#pragma unroll
                for (int T = 0; T < 2; ++T)
#pragma unroll
                    for (int s = 0; s < NS; ++s)
                        kr[e][T][s] = buffer_stream16(kp + kbase[T], kPageBytes, k_lane,
                                                      to_bytes(tile_el(T) + ((uint32_t)s << (BS + 5))));
                const uint16_t *vp = static_cast<const uint16_t *>(vpool);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    if constexpr (HALF) {
                        const size_t vbase = g4 < 2 ? kbase[0] : kbase[1];
                        vr[e][dt] = load_stream16(vp + vbase + value_offset(8 * (g4 & 1), 16 * dt + h, D, BS));
                    } else {
                        vr[e][dt] = buffer_stream16(vp + kbase[0], kPageBytes, v_lane, to_bytes(blk + 512u * dt));
                    }
                }
            }
            // keep the block's loads ahead of the compute that follows them
            __builtin_amdgcn_sched_barrier(0);
        };
        // ---- online softmax and PV of block i from ring slot e.  A block that
        // needs no keys is computed fully masked with its values zeroed (its slot
        // holds another block's data); there is no branch around it, so the
        // compiler keeps every ring load where it is issued.
        auto consume = [&](int e, int i) __attribute__((always_inline)) {
            // the page slot of each tile (for the int4 scale and zero point)
            const int jt[2] = {HALF ? 2 * i : i / NB, HALF ? 2 * i + 1 : i / NB};
            // scores of the 32 keys (two 16-row tiles)
            floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                bf16x8 k0, k1;
                if constexpr (I4) {
                    const uint32_t w0 = pick(kr[e][0][0], s), w1 = pick(kr[e][1][0], s);
                    k0 = __builtin_bit_cast(bf16x8, nibbles_bf16x8_split(w0));
                    k1 = __builtin_bit_cast(bf16x8, nibbles_bf16x8_split(w1));
                } else {
                    k0 = __builtin_bit_cast(bf16x8, kr[e][0][s]);
                    k1 = __builtin_bit_cast(bf16x8, kr[e][1][s]);
                }
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb[s], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb[s], s1, 0, 0, 0);
            }
            // lane holds the logits of head h for tokens 4*g4 + r (x[r]) and
            // 16 + 4*g4 + r (x[4 + r]) of the block, r = 0..3
            float x[8];
            if constexpr (I4) {
                // (s - off) * sc as one fma per logit, with off * sc formed once per tile
                const float sc0 = sk[jt[0]] * a.scale_log2, sc1 = sk[jt[1]] * a.scale_log2;
                const float noff0 = -((128.f + zk[jt[0]]) * qsum) * sc0, noff1 = -((128.f + zk[jt[1]]) * qsum) * sc1;
#pragma unroll
                for (int r = 0; r < 4; ++r) { x[r] = fmaf(s0[r], sc0, noff0); x[4 + r] = fmaf(s1[r], sc1, noff1); }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) { x[r] = s0[r] * a.scale_log2; x[4 + r] = s1[r] * a.scale_log2; }
            }
            const bool full = (full_bits >> i) & 1u;
            if (!full) {                        // (wavefront-uniform branch)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int T = jj >> 2;
                    const bool vis = need_t(i, T) & token_visible(a, w, tok_of(i, T) + 4 * g4 + (jj & 3));
                    x[jj] = vis ? x[jj] : -__builtin_inff();
                }
            }
            float mb = -__builtin_inff();
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) mb = fmaxf(mb, x[jj]);
            mb = max_xor32(max_xor16(mb));
            const float m_new = fmaxf(m_run, mb);
            // reference of the exponentials: any finite value while nothing is visible yet
            const float m_ref = m_new == -__builtin_inff() ? 0.f : m_new;
            const float alpha = exp2_fast(m_run - m_ref);
            float psum = 0.f, fed[2] = {0.f, 0.f};
            uint32_t pk[4];
#pragma unroll
            for (int jj = 0; jj < 8; jj += 2) {
                const float pa = exp2_fast(x[jj] - m_ref);
                const float pb = exp2_fast(x[jj + 1] - m_ref);
                psum += pa + pb;
                // v_cvt_pk_bf16_f32: round to nearest even
                uint32_t u;
                if constexpr (I4) {
                    const float svt = sv[jt[jj >> 2]];
                    u = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{pa * svt, pb * svt}, bf16x2));
                    // the two fed weights, summed by one v_dot2 against (1, 1)
                    fed[jj >> 2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u),
                                                                   __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                                                   fed[jj >> 2], false);
                } else {
                    u = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{pa, pb}, bf16x2));
                }
                pk[jj / 2] = u;
            }
            l_run = l_run * alpha + psum;
            if constexpr (I4) corr = corr * alpha + (128.f + zv[jt[0]]) * fed[0] + (128.f + zv[jt[1]]) * fed[1];
            m_run = m_new;
            // The PV operand of lane (h, g4) wants tokens 8*g4 .. 8*g4 + 7.  Swapping
            // the upper 32 lanes of pk[0..1] (tokens 4*g4 + r) with the lower 32
            // lanes of pk[2..3] (tokens 16 + 4*g4 + r), then the odd 16-lane rows
            // of the first result with the even rows of the second, regroups the
            // four 4-token runs of every head into that order.
            uint32_t pv[4];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const auto r32 = __builtin_amdgcn_permlane32_swap(pk[d], pk[2 + d], false, false);
                const auto r16 = __builtin_amdgcn_permlane16_swap(r32[0], r32[1], false, false);
                pv[d] = r16[0];
                pv[2 + d] = r16[1];
            }
            // int4: the unpacked values come in the token order 0 2 4 6 1 3 5 7
            const bf16x8 pbv = __builtin_bit_cast(bf16x8, I4 ? split_order(pv[0], pv[1], pv[2], pv[3])
                                                             : make_uint4(pv[0], pv[1], pv[2], pv[3]));
            // bf16 value slots after the current token may hold any bits: zero them
            // so a zero probability never meets a NaN in the PV product (int4 codes
            // always unpack to finite values)
            if constexpr (!I4) {
                const bool tail =
                    !full && (!(need_t(i, 0) & need_t(i, 1)) || max(tok_of(i, 0), tok_of(i, 1)) + 15 > w.t_pool);
                if (tail) {                     // (wavefront-uniform branch: masks the ring slot in place)
                    const int vt = HALF ? g4 >> 1 : 0;   // the tile whose tokens this lane's value rows hold
                    const int nvalid =
                        ((need_bits >> (2 * i + vt)) & 1u) ? w.t_pool - ((vt ? tok_of(i, 1) : tok_of(i, 0)) + (HALF ? 8 * (g4 & 1) : 8 * g4)) + 1 : 0;
                    uint32_t keep[4];
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2)
                        keep[q2] = (2 * q2 < nvalid ? 0x0000FFFFu : 0u) | (2 * q2 + 1 < nvalid ? 0xFFFF0000u : 0u);
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        vr[e][dt].x &= keep[0]; vr[e][dt].y &= keep[1];
                        vr[e][dt].z &= keep[2]; vr[e][dt].w &= keep[3];
                    }
                }
            }
            // rescale the accumulators only when some head's running maximum moved
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
            }
            // int4 rows -> per-tile dwords: before, lane group q's slot c holds
            // dword c (tokens 8c ..) of channel 16 * (VRW * q + j) + h; after the
            // swaps lane group g4's slot q holds dword g4 of that same channel,
            // i.e. the operand of tile VRW * q + j
            uint32_t vy[I4 && !HALF ? NDT : 1];
            if constexpr (I4 && !HALF) {
#pragma unroll
                for (int j = 0; j < VRW; ++j) {
                    uint32_t d[4] = {vq[e][j].x, vq[e][j].y, vq[e][j].z, vq[e][j].w};
                    swap_halves32(d[0], d[2]);
                    swap_halves32(d[1], d[3]);
                    swap_rows16(d[0], d[1]);
                    swap_rows16(d[2], d[3]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) vy[VRW * q + j] = d[q];
                }
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                uint4 va;
                if constexpr (I4) {
                    // 4 bytes = tokens 8*g4 .. 8*g4+7 of channel 16*dt + h
                    va = nibbles_bf16x8_split(HALF ? vr4[e][dt] : vy[dt]);
                } else {
                    va = vr[e][dt];
                }
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pbv, o[dt], 0, 0, 0);
            }
        };
        // ---- the ring: BIF blocks in flight
#pragma unroll
        for (int i = 0; i < BIF; ++i) issue(i, i);
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            consume(i % BIF, i);
            if (i + BIF < NBW) issue(i % BIF, i + BIF);
        }
    }
    l_run = sum_xor32(sum_xor16(l_run));
    if constexpr (I4) {
        // the head's correction sums the four lane groups' tokens
        corr = sum_xor32(sum_xor16(corr));
    }

    float *my = lds + wave * (32 + 16 * D);
    if (g4 == 0) { my[h] = m_run; my[16 + h] = l_run; }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) my[32 + h * D + 16 * dt + 4 * g4 + r] = o[dt][r] - corr;
    if (a.stats && !a.k_new && !w.streaming && w.chunk == 0 && wave == 0) refresh_current_stats(a, w, KVT);
    if (j_new >= 0) {
        // token t as a one-token partial state (log2-domain logit per head, its
        // value row) next to the wavefronts' states, then written to its page
        float sk_n = 1.f, zk_n = 0.f, sv_n = 1.f, zv_n = 0.f;
        if constexpr (I4) {
            sk_n = fp16_bits_to_f32(uint16_t(ksz_n)); zk_n = fp16_bits_to_f32(uint16_t(ksz_n >> 16));
            sv_n = fp16_bits_to_f32(uint16_t(vsz_n)); zv_n = fp16_bits_to_f32(uint16_t(vsz_n >> 16));
        }
        float dot = 0.f;
        if constexpr (I4) {
            // this lane's codes: channels (D/4)*g4 .. + D/4 - 1, the order of qb
            const uint4 kc = D == 128 ? s_new[g4]
                                      : make_uint4(reinterpret_cast<const uint2 *>(s_new)[g4].x,
                                                   reinterpret_cast<const uint2 *>(s_new)[g4].y, 0u, 0u);
            const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4 qraw = opaque(__builtin_bit_cast(uint4, qb[s]));
                const uint32_t qw[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int c = 8 * s + (j < 4 ? 2 * j : 2 * j - 7);   // code c of the lane's run (qb order)
                    const float kj = (float)((kw[c / 8] >> (4 * (c % 8))) & 15u) - zk_n;
                    dot = fmaf((j & 1) ? bf16_hi(qw[j / 2]) : bf16_lo(qw[j / 2]), kj, dot);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const uint4 qraw = opaque(__builtin_bit_cast(uint4, qb[s])), kraw = s_new[4 * s + g4];   // channels 32s + 8*g4 ..
                const uint32_t qw[4] = {qraw.x, qraw.y, qraw.z, qraw.w}, kw[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    dot = fmaf((j & 1) ? bf16_hi(qw[j / 2]) : bf16_lo(qw[j / 2]),
                               (j & 1) ? bf16_hi(kw[j / 2]) : bf16_lo(kw[j / 2]), dot);
            }
        }
        dot = sum_xor32(sum_xor16(dot));
        float *nt = lds + kDecodeWaves * (32 + 16 * D);
        if (g4 == 0) nt[h] = dot * sk_n * a.scale_log2;
        for (int c = lane; c < D; c += kWave) {
            float vc;
            if constexpr (I4) vc = ((float)((s_new8[kNewRow + c / 2] >> (4 * (c & 1))) & 15u) - zv_n) * sv_n;
            else vc = bf16_to_f32(*reinterpret_cast<const uint16_t *>(s_new8 + kNewRow + 2 * c));
            nt[16 + c] = vc;
        }
        append_write<KVT, D, NP, PPW>(a, w, j_new, hp, pg, kpool, vpool, kszp, vszp, ksz_n, vsz_n, s_new8, lane);
    }
    __syncthreads();
    merge_waves_and_store<kDecodeWaves>(a, w, lds, D, a.k_new != nullptr);
    finish_head<uint16_t, kDecodeMergeBatch>(a, w, D);
}

// ---------------------------------------------------------------------------
// f32 K/V, f32 q: plain VALU path (lanes own tokens for QK^T, channels for PV)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeArgs a) {
    extern __shared__ float lds[];
    WorkItem w = decode_item(a);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int G = a.group, NP = a.page_size;
    constexpr int CPL = D / 64;                   // channels per lane in PV
    __shared__ int s_list[kListSlots];
    if (wave == 0) wg_pages<4>(a, w, s_list);

    float *qs = lds + 4 * (32 + 16 * D);          // [G][D]
    float *ps = qs + 16 * D + wave * 16 * 64;     // this wave's [16][64] probabilities
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x)
        qs[idx] = static_cast<const float *>(a.q)[((size_t)w.b * a.num_q_heads + (size_t)w.kv * G) * D + idx];
    __syncthreads();
    w.t = s_list[0];
    w.L = s_list[1];
    w.t_pool = w.t;                                // (the f32 path substitutes the new token itself)
    const int my_page = s_list[2 + wave], my_pool = s_list[6 + wave];

    float o[16][CPL];
    float m_run[16], l_run[16];
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
        m_run[hh] = -__builtin_inff();
        l_run[hh] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[hh][c] = 0.f;
    }

    const bool in_cache = w.streaming && a.sc_k != nullptr;
    const float *kpool = static_cast<const float *>(in_cache ? a.sc_k : a.k);
    const float *vpool = static_cast<const float *>(in_cache ? a.sc_v : a.v);
    const int bs = block_shift(NP);

    // fused append: this wavefront reads the page of token t and takes the
    // token from the new rows (its page does not hold it yet), then writes it
    const bool put_new = a.k_new != nullptr && my_page >= 0 && my_page == w.t / NP;
    const size_t new_row = ((size_t)w.b * a.num_kv_heads + w.kv) * D;
    const float *k_new = static_cast<const float *>(a.k_new) + new_row;
    const float *v_new = static_cast<const float *>(a.v_new) + new_row;

    if (my_page >= 0) {
        const int page = my_page;
        const size_t head_page = in_cache ? (size_t)my_pool : (size_t)my_pool * a.hm.pool_heads + pool_slot(a.hm, w.kv);
        const float *kp = kpool + head_page * NP * D;
        const float *vp = vpool + head_page * NP * D;
        for (int s0 = 0; s0 < NP; s0 += kWave) {
            const int slot = s0 + lane;
            const int p = page * NP + slot;
            const bool vis = slot < NP && token_visible(a, w, p);
            float sc[16];
#pragma unroll
            for (int hh = 0; hh < 16; ++hh) sc[hh] = 0.f;
            if (slot < NP) {
                const bool mine = put_new && p == w.t;
                for (int d = 0; d < D; d += 4) {
                    const float4 kv4 = *reinterpret_cast<const float4 *>(mine ? k_new + d
                                                                               : kp + key_offset(slot, d, D, bs));
#pragma unroll
                    for (int hh = 0; hh < 16; ++hh) {
                        if (hh < G) {
                            const float *qh = qs + hh * D + d;
                            sc[hh] = fmaf(kv4.x, qh[0], sc[hh]);
                            sc[hh] = fmaf(kv4.y, qh[1], sc[hh]);
                            sc[hh] = fmaf(kv4.z, qh[2], sc[hh]);
                            sc[hh] = fmaf(kv4.w, qh[3], sc[hh]);
                        }
                    }
                }
            }
            float alpha[16];
#pragma unroll
            for (int hh = 0; hh < 16; ++hh) {
                if (hh >= G) { alpha[hh] = 1.f; continue; }
                const float x = vis ? sc[hh] * a.scale_log2 : -__builtin_inff();
                const float mb = wave_max(x);
                if (mb == -__builtin_inff()) { alpha[hh] = 1.f; ps[hh * 64 + lane] = 0.f; continue; }
                const float m_new = fmaxf(m_run[hh], mb);
                alpha[hh] = exp2_fast(m_run[hh] - m_new);
                const float pr = vis ? exp2_fast(x - m_new) : 0.f;
                const float psum = wave_sum(pr);
                l_run[hh] = l_run[hh] * alpha[hh] + psum;
                m_run[hh] = m_new;
                ps[hh * 64 + lane] = pr;
            }
            __builtin_amdgcn_wave_barrier();
            const int nslots = max(0, min(min(kWave, NP - s0), w.t - (page * NP + s0) + 1));
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int d = lane * CPL + c;

                float acc[16];
#pragma unroll
                for (int hh = 0; hh < 16; ++hh) acc[hh] = o[hh][c] * alpha[hh];
                for (int sl = 0; sl < nslots; ++sl) {
                    const float vv = put_new && page * NP + s0 + sl == w.t ? v_new[d]
                                                                           : vp[value_offset(s0 + sl, d, D, bs)];
#pragma unroll
                    for (int hh = 0; hh < 16; ++hh)
                        if (hh < G) acc[hh] = fmaf(ps[hh * 64 + sl], vv, acc[hh]);
                }
#pragma unroll
                for (int hh = 0; hh < 16; ++hh) o[hh][c] = acc[hh];
            }
            __builtin_amdgcn_wave_barrier();
        }
    }

    if (put_new) {
        // the token into its page, and into its logical page's statistics
        const size_t head_page = in_cache ? (size_t)my_pool : (size_t)my_pool * a.hm.pool_heads + pool_slot(a.hm, w.kv);
        float *kp = const_cast<float *>(kpool) + head_page * NP * D;
        float *vp = const_cast<float *>(vpool) + head_page * NP * D;
        const int slot = w.t % NP, NL = a.logical_page, jl = slot / NL, g = NP / NL;
        const bool opens = slot % NL == 0;
        float *st = static_cast<float *>(a.stats) + ((head_page * g + jl) * 2) * D;
        for (int c = lane; c < D; c += kWave) {
            const float x = k_new[c];
            kp[key_offset(slot, c, D, bs)] = x;
            vp[value_offset(slot, c, D, bs)] = v_new[c];
            if (a.stats && !w.streaming) {
                st[c] = opens ? x : fminf(st[c], x);
                st[D + c] = opens ? x : fmaxf(st[D + c], x);
            }
        }
    }

    float *my = lds + wave * (32 + 16 * D);
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
        if (lane == 0) { my[hh] = m_run[hh]; my[16 + hh] = l_run[hh]; }
#pragma unroll
        for (int c = 0; c < CPL; ++c) my[32 + hh * D + lane * CPL + c] = o[hh][c];
    }
    if (a.stats && !a.k_new && !w.streaming && w.chunk == 0 && wave == 0) refresh_current_stats(a, w, LSA_F32);
    __syncthreads();
    merge_waves_and_store<4>(a, w, lds, D, false);
    finish_head<float, 17>(a, w, D);
}

}  // namespace

namespace {

template <int D, int KVT>
hipError_t launch_mfma(const DecodeArgs &a, unsigned grid, hipStream_t s) {
    // the wavefronts' states, then the appended token's one-token state
    const size_t lds = (kDecodeWaves * (32 + 16 * (size_t)D) + 16 + D) * sizeof(float);
    const dim3 block(kDecodeWaves * kWave);
    switch (a.page_size) {
        case 16: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 16>), dim3(grid), block, lds, s, a); break;
        case 32: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 32>), dim3(grid), block, lds, s, a); break;
        case 64: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 64>), dim3(grid), block, lds, s, a); break;
        case 128: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 128>), dim3(grid), block, lds, s, a); break;
        case 256: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 256>), dim3(grid), block, lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int q_dtype, int kv_dtype, hipStream_t s) {
    const long long grid = (long long)a.batch * a.chunks_per_seq;
    if (grid == 0) return hipSuccess;
    hipError_t e = hipSuccess;
    if (q_dtype == LSA_BF16 && kv_dtype == LSA_BF16) {
        e = a.head_dim == 128 ? launch_mfma<128, LSA_BF16>(a, (unsigned)grid, s)
                              : launch_mfma<64, LSA_BF16>(a, (unsigned)grid, s);
    } else if (q_dtype == LSA_BF16 && kv_dtype == LSA_INT4) {
        e = a.head_dim == 128 ? launch_mfma<128, LSA_INT4>(a, (unsigned)grid, s)
                              : launch_mfma<64, LSA_INT4>(a, (unsigned)grid, s);
    } else if (q_dtype == LSA_F32 && kv_dtype == LSA_F32) {
        const size_t lds = (4 * (32 + 16 * (size_t)a.head_dim) + 16 * (size_t)a.head_dim + 4 * 16 * 64) * sizeof(float);
        if (a.head_dim == 128)
            hipLaunchKernelGGL(decode_f32_kernel<128>, dim3((unsigned)grid), dim3(256), lds, s, a);
        else
            hipLaunchKernelGGL(decode_f32_kernel<64>, dim3((unsigned)grid), dim3(256), lds, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace lsa
