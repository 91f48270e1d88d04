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
// runs four wavefronts of 128 tokens each (eight pages of 64 tokens per chunk);
// the f32 path four wavefronts of one page.  The last workgroup of a
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
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct WorkItem {
    int b, kv, chunk, t, L;
    bool streaming;
};

__device__ __forceinline__ WorkItem decode_item(const DecodeArgs &a) {
    WorkItem w;
    w.b = blockIdx.x / a.chunks_per_seq;
    int off = blockIdx.x % a.chunks_per_seq;
    int kv = 0;
    for (; kv < a.num_kv_heads; ++kv) {
        const int c = a.kind[kv] ? a.chunks_str : a.chunks_ret;
        if (off < c) break;
        off -= c;
    }
    w.kv = kv;
    w.chunk = off;
    w.streaming = a.kind[kv] != 0;
    return w;
}

// Slots of the per-workgroup page list in LDS: t, L, then the sequence pages
// of the chunk, then their pool pages (-1: no page).
constexpr int kListSlots = 2 + 2 * kMaxChunkPages;

// Wavefront 0 of a workgroup resolves the CP pages of its chunk: the attended
// pages of a (sequence, KV head) in ascending order are the selection row
// (valid entries first, then -1) followed by the current page when the row
// lacks it (retrieval heads), or the sink pages followed by the local window
// (streaming heads); the chunk takes list entries CP * chunk .. CP * chunk + CP - 1.
// seq_lens and the selection entries are loaded together, then the CP
// page-table entries: two dependent loads in all.
template <int CP>
__device__ __forceinline__ void wg_pages(const DecodeArgs &a, const WorkItem &w, int *list) {
    static_assert(CP <= kMaxChunkPages && (CP & (CP - 1)) == 0, "chunk pages");
    const int lane = threadIdx.x % kWave;
    const int NP = a.page_size;
    const int i = w.chunk * CP + (lane & (CP - 1));    // list index of this lane's page (lanes 0..CP-1)
    const int32_t *sel = w.streaming ? nullptr : a.selected + ((size_t)w.b * a.num_kv_heads + w.kv) * a.sel_k;
    int m_row = -1, m_i = -1;
    if (sel) {
        if (lane < a.sel_k) m_row = sel[lane];
        if (lane < CP && i < a.sel_k) m_i = sel[i];
    }
    const int L = a.seq_lens[w.b];
    const int t = L - 1, cur = t / NP;
    int page = -1;
    if (w.streaming) {
        const int sink_end = min(a.sink, t + 1);          // tokens [0, sink_end)
        const int n_sink = (sink_end + NP - 1) / NP;
        const int local_first = max(max(0, t - a.local + 1) / NP, n_sink);
        const int n = n_sink + max(0, cur - local_first + 1);
        if (i < n) page = i < n_sink ? i : local_first + (i - n_sink);
    } else {
        int cnt = __popcll(__ballot(m_row >= 0));
        bool in = __ballot(m_row == cur) != 0;
        for (int j0 = kWave; j0 < a.sel_k; j0 += kWave) {
            const int m = j0 + lane < a.sel_k ? sel[j0 + lane] : -1;
            cnt += __popcll(__ballot(m >= 0));
            in |= __ballot(m == cur) != 0;
        }
        const int n = cnt + (in ? 0 : 1);
        if (i < n) page = i < cnt ? m_i : cur;
    }
    int pool = -1;
    if (lane < CP && page >= 0) pool = a.page_table[(size_t)w.b * a.max_pages + page];
    if (lane == 0) { list[0] = t; list[1] = L; }
    if (lane < CP) { list[2 + lane] = page; list[2 + CP + lane] = pool; }
}

__device__ __forceinline__ bool token_visible(const DecodeArgs &a, const WorkItem &w, int p) {
    // bitwise, not short-circuit: no branch inside the block compute
    return (p <= w.t) & (!w.streaming | (p < a.sink) | ((w.t - p) < a.local));
}

// Does the 32-token block starting at tok0 hold any attended token?
__device__ __forceinline__ bool block_needed(const DecodeArgs &a, const WorkItem &w, int tok0) {
    if (tok0 > w.t) return false;
    if (!w.streaming) return true;
    const int p_last = min(tok0 + 31, w.t);
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
    const size_t hp = (size_t)pool * a.num_kv_heads + w.kv;
    const size_t page_base = hp * NP * D;
    if (kv_dtype == LSA_INT4) {
        if (lane >= D / 2) return;
        const uint8_t *k = static_cast<const uint8_t *>(a.k);
        uint32_t lo_min = 15, lo_max = 0, hi_min = 15, hi_max = 0;
        for (int r = 0; r < rows; ++r) {
            const uint32_t byte = k[(page_base + key_offset(row0 + r, 2 * lane, D)) / 2];
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
            const size_t off = page_base + key_offset(row0 + r, ch, D);
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
template <int NW>
__device__ __forceinline__ void merge_waves_and_store(const DecodeArgs &a, const WorkItem &w,
                                                      const float *lds, int D) {
    const int G = a.group;
    const int wave_stride = 32 + 16 * D;
    const size_t rec_size = 32 + (size_t)G * D;
    float *rec = a.part + (((size_t)w.b * a.num_kv_heads + w.kv) * a.chunks_max + w.chunk) * rec_size;
    for (int pi = threadIdx.x; pi < G * D / 2; pi += blockDim.x) {
        const int h = (2 * pi) / D, d = 2 * pi - h * D;
        float M = -__builtin_inff();
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, lds[wv * wave_stride + h]);
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

// The eight codes of `w` as bf16 bit patterns 0x4300 | c (= 128 + c): dword
// k holds the low nibble of byte k in its low half and the high nibble in its
// high half.  The low and high nibbles are masked out once; one byte permute
// per dword then places byte k of each in bytes 0 and 2 (bytes 1 and 3 zero,
// selector 12), and one OR sets the exponent bytes.
__device__ __forceinline__ uint4 nibbles_bf16x8(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    // v_perm_b32 selector bytes: 0..3 pick bytes of the second operand (lo),
    // 4..7 bytes of the first (hi), 12 gives 0x00
    return make_uint4(__builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x43004300u,
                      __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x43004300u,
                      __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x43004300u,
                      __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x43004300u);
}

__device__ __forceinline__ uint32_t pick(const uint4 &u, int i) {
    return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// ---------------------------------------------------------------------------
// MFMA kernel, bf16 or int4 pool, bf16 q
// ---------------------------------------------------------------------------
template <int D, int KVT, int NB>
__global__ __launch_bounds__(kDecodeWaves * kWave, 2) void decode_mfma_kernel(DecodeArgs a) {
    constexpr bool I4 = KVT == LSA_INT4;
    constexpr int NS = D / 32;            // MFMA k-steps over channels
    constexpr int NDT = D / 16;           // output channel tiles
    constexpr int NP = 32 * NB;           // page size
    constexpr int PPW = decode_pages_per_wave(KVT, NP);
    constexpr int NBW = PPW * NB;         // 32-token blocks per wavefront
    constexpr int CP = kDecodeWaves * PPW;
    constexpr int BIF = I4 ? (NBW < 4 ? NBW : 4) : 2;   // blocks in flight (ring size)
    extern __shared__ float lds[];
    WorkItem w = decode_item(a);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int h = lane & 15, g4 = lane >> 4;
    const int G = a.group;

    // B operand of QK^T: column h = query head.  bf16 pools: step s holds
    // channels 32s + 8*g4 + j; int4 pools: channels (D/4)*g4 + 8s + j, so that a
    // lane's steps cover one contiguous run of codes of its key row.
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
            }
            qb[s] = __builtin_bit_cast(bf16x8, raw);
        }
        if constexpr (I4) {
            qsum = sum_xor32(sum_xor16(qsum));
        }
    }
    __shared__ int s_list[kListSlots];
    if (wave == 0) wg_pages<CP>(a, w, s_list);
    __syncthreads();
    w.t = __builtin_amdgcn_readfirstlane(s_list[0]);
    w.L = __builtin_amdgcn_readfirstlane(s_list[1]);

    // this wavefront's pages: chunk slots PPW*wave .. PPW*wave + PPW - 1
    int pg[PPW];
    size_t hp[PPW];
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
        pg[j] = __builtin_amdgcn_readfirstlane(s_list[2 + PPW * wave + j]);
        const int pool = __builtin_amdgcn_readfirstlane(s_list[2 + CP + PPW * wave + j]);
        hp[j] = (size_t)max(pool, 0) * a.num_kv_heads + w.kv;
    }
    // block i of the wavefront: page slot i / NB, 32-token block i % NB of that page
    bool need[NBW];
    bool any = false;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        need[i] = pg[i / NB] >= 0 && block_needed(a, w, pg[i / NB] * NP + 32 * (i % NB));
        any |= need[i];
    }

    floatx4 o[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff(), l_run = 0.f;
    float corr = 0.f;                      // int4: (128 + z_v) * sum of fed weights (per lane)

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
                    const uint32_t ksz = *reinterpret_cast<const uint32_t *>(a.k_sz + hp[j] * 2);
                    const uint32_t vsz = *reinterpret_cast<const uint32_t *>(a.v_sz + hp[j] * 2);
                    sk[j] = fp16_bits_to_f32(uint16_t(ksz)); zk[j] = fp16_bits_to_f32(uint16_t(ksz >> 16));
                    sv[j] = fp16_bits_to_f32(uint16_t(vsz)); zv[j] = fp16_bits_to_f32(uint16_t(vsz >> 16));
                }
            }
        }
        // source of each ring load: the block itself, or the first needed block
        size_t src_hp[NBW];
        int src_kb[NBW];
        {
            size_t f_hp = 0;
            int f_kb = 0;
            bool found = false;
#pragma unroll
            for (int i = 0; i < NBW; ++i)
                if (need[i] && !found) { f_hp = hp[i / NB]; f_kb = i % NB; found = true; }
#pragma unroll
            for (int i = 0; i < NBW; ++i) {
                src_hp[i] = need[i] ? hp[i / NB] : f_hp;
                src_kb[i] = need[i] ? i % NB : f_kb;
            }
        }

        uint4 kr[BIF][2][I4 ? 1 : NS];
        uint4 vr[BIF][I4 ? 1 : NDT];
        uint32_t vr4[BIF][I4 ? NDT : 1];
        // ---- issue every K and V load of block i into ring slot e
        auto issue = [&](int e, int i) {
            const size_t base = src_hp[i] * NP * D;
            const int kb = src_kb[i];
            if constexpr (I4) {
                const uint8_t *k8 = static_cast<const uint8_t *>(a.k);
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    const uint8_t *row = k8 + (base + key_offset(32 * kb + 16 * T + rho, (D / 4) * g4, D)) / 2;
                    if constexpr (D == 128) {
                        kr[e][T][0] = load_stream16(row);
                    } else {
                        const uint2 u = load_stream8(row);
                        kr[e][T][0] = make_uint4(u.x, u.y, 0, 0);
                    }
                }
                const uint8_t *v8 = static_cast<const uint8_t *>(a.v);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    vr4[e][dt] = load_stream4(v8 + (base + value_offset(32 * kb + 8 * g4, 16 * dt + h, D)) / 2);
            } else {
                const uint16_t *kp = static_cast<const uint16_t *>(a.k) + base;
#pragma unroll
                for (int T = 0; T < 2; ++T)
#pragma unroll
                    for (int s = 0; s < NS; ++s)
                        kr[e][T][s] = load_stream16(kp + key_offset(32 * kb + 16 * T + rho, 32 * s + 8 * g4, D));
                const uint16_t *vp = static_cast<const uint16_t *>(a.v) + base;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    vr[e][dt] = load_stream16(vp + value_offset(32 * kb + 8 * g4, 16 * dt + h, D));
            }
            // keep the block's loads ahead of the compute that follows them
            __builtin_amdgcn_sched_barrier(0);
        };
        // ---- online softmax and PV of block i from ring slot e.  A block that
        // needs no keys is computed fully masked with its values zeroed (its slot
        // holds another block's data); there is no branch around it, so the
        // compiler keeps every ring load where it is issued.
        auto consume = [&](int e, int i) {
            const bool blk = need[i];
            const int j = i / NB;
            const int tok0 = pg[j] * NP + 32 * (i % NB);
            // scores of the 32 keys (two 16-row tiles)
            floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                bf16x8 k0, k1;
                if constexpr (I4) {
                    const uint32_t w0 = pick(kr[e][0][0], s), w1 = pick(kr[e][1][0], s);
                    k0 = __builtin_bit_cast(bf16x8, nibbles_bf16x8(w0));
                    k1 = __builtin_bit_cast(bf16x8, nibbles_bf16x8(w1));
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
                const float off = (128.f + zk[j]) * qsum;
                const float sc = sk[j] * a.scale_log2;
#pragma unroll
                for (int r = 0; r < 4; ++r) { x[r] = (s0[r] - off) * sc; x[4 + r] = (s1[r] - off) * sc; }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) { x[r] = s0[r] * a.scale_log2; x[4 + r] = s1[r] * a.scale_log2; }
            }
            float mb = -__builtin_inff();
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const bool vis = blk & token_visible(a, w, tok0 + 4 * g4 + (jj & 3) + 16 * (jj >> 2));
                x[jj] = vis ? x[jj] : -__builtin_inff();        // a select, not a branch
                mb = fmaxf(mb, x[jj]);
            }
            mb = max_xor32(max_xor16(mb));
            const float m_new = fmaxf(m_run, mb);
            // reference of the exponentials: any finite value while nothing is visible yet
            const float m_ref = m_new == -__builtin_inff() ? 0.f : m_new;
            const float alpha = exp2_fast(m_run - m_ref);
            float psum = 0.f, fed = 0.f;
            uint32_t pk[4];
#pragma unroll
            for (int jj = 0; jj < 8; jj += 2) {
                const float pa = exp2_fast(x[jj] - m_ref);
                const float pb = exp2_fast(x[jj + 1] - m_ref);
                psum += pa + pb;
                uint16_t ba, bb;
                if constexpr (I4) {
                    ba = f32_to_bf16_rne(pa * sv[j]);
                    bb = f32_to_bf16_rne(pb * sv[j]);
                    fed += bf16_to_f32(ba) + bf16_to_f32(bb);
                } else {
                    ba = f32_to_bf16_rne(pa);
                    bb = f32_to_bf16_rne(pb);
                }
                pk[jj / 2] = uint32_t(ba) | (uint32_t(bb) << 16);
            }
            l_run = l_run * alpha + psum;
            if constexpr (I4) corr = corr * alpha + (128.f + zv[j]) * fed;
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
            const bf16x8 pbv = __builtin_bit_cast(bf16x8, make_uint4(pv[0], pv[1], pv[2], pv[3]));
            // slots after the current token may hold any bits: zero their values so a
            // zero probability never meets a NaN in the PV product
            const bool tail = !blk || tok0 + 31 > w.t;
            const int nvalid = blk ? w.t - (tok0 + 8 * g4) + 1 : 0;
            uint32_t keep[4] = {~0u, ~0u, ~0u, ~0u};
            if (tail) {
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2)
                    keep[q2] = (2 * q2 < nvalid ? 0x0000FFFFu : 0u) | (2 * q2 + 1 < nvalid ? 0xFFFF0000u : 0u);
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                uint4 va;
                if constexpr (I4) {
                    // 4 bytes = tokens 8*g4 .. 8*g4+7 of channel 16*dt + h
                    const uint32_t wv4 = vr4[e][dt];
                    va = nibbles_bf16x8(wv4);
                } else {
                    va = vr[e][dt];
                }
                if (tail) {
                    va.x &= keep[0]; va.y &= keep[1]; va.z &= keep[2]; va.w &= keep[3];
                }
                o[dt] *= alpha;
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
    if (a.stats && !w.streaming && w.chunk == 0 && wave == 0) refresh_current_stats(a, w, KVT);
    __syncthreads();
    merge_waves_and_store<kDecodeWaves>(a, w, lds, D);
    // one batch of records covers a 4096-token budget (its pages plus the current one)
    constexpr int CB = (4096 / NP + CP) / CP < 17 ? (4096 / NP + CP) / CP : 17;
    finish_head<uint16_t, CB>(a, w, D);
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

    const float *kpool = static_cast<const float *>(a.k);
    const float *vpool = static_cast<const float *>(a.v);

    if (my_page >= 0) {
        const int page = my_page;
        const size_t head_page = (size_t)my_pool * a.num_kv_heads + w.kv;
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
                for (int d = 0; d < D; d += 4) {
                    const float4 kv4 = *reinterpret_cast<const float4 *>(kp + key_offset(slot, d, D));
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
                    const float vv = vp[value_offset(s0 + sl, d, D)];
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

    float *my = lds + wave * (32 + 16 * D);
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
        if (lane == 0) { my[hh] = m_run[hh]; my[16 + hh] = l_run[hh]; }
#pragma unroll
        for (int c = 0; c < CPL; ++c) my[32 + hh * D + lane * CPL + c] = o[hh][c];
    }
    if (a.stats && !w.streaming && w.chunk == 0 && wave == 0) refresh_current_stats(a, w, LSA_F32);
    __syncthreads();
    merge_waves_and_store<4>(a, w, lds, D);
    finish_head<float, 17>(a, w, D);
}

}  // namespace

namespace {

template <int D, int KVT>
hipError_t launch_mfma(const DecodeArgs &a, unsigned grid, hipStream_t s) {
    const size_t lds = kDecodeWaves * (32 + 16 * (size_t)D) * sizeof(float);
    const dim3 block(kDecodeWaves * kWave);
    switch (a.page_size) {
        case 32: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 1>), dim3(grid), block, lds, s, a); break;
        case 64: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 2>), dim3(grid), block, lds, s, a); break;
        case 128: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 4>), dim3(grid), block, lds, s, a); break;
        case 256: hipLaunchKernelGGL((decode_mfma_kernel<D, KVT, 8>), dim3(grid), block, lds, s, a); break;
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
