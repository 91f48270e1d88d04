// Query-aware page scoring, logical -> physical max reduction, and top-K
// selection (LServe explainer, 技術的詳細 / 動的スパーシティ: the score
// S^j = sum_i max(q[i] k_max^j[i], q[i] k_min^j[i]); 階層的ページング:
// physical importance = max over its logical pages; figure: top-K physical
// pages; abstract page: a constant page budget).
//
// Scoring.  For a query head h, max(q_h[i] k_max[i], q_h[i] k_min[i]) equals
// q+_h[i] k_max[i] + q-_h[i] k_min[i] with q+ = max(q, 0), q- = min(q, 0).
// Summed over the G heads of a GQA group this is
//     S^j = sum_i Qp[i] k_max^j[i] + Qn[i] k_min^j[i],
//     Qp = sum_h max(q_h, 0),  Qn = sum_h min(q_h, 0),
// the same real number with one product pair per channel instead of G.  Qp,
// Qn and the sums are formed in fp64 (the products of bf16/f32 operands are
// exact there), so S^j and P_m carry only fp64 rounding and the ranking is
// decided in fp64.  For int4 keys k = (c - z) s with one (s, z) per physical
// page and head, S^j = s * (sum_i Qp c_max + Qn c_min - z * sum_i (Qp + Qn)).
// A group of lanes owns one logical page (one 16-byte load of its minima and
// one of its maxima per lane); the logical page that holds the current token
// is scored from the keys themselves.  Logical scores go to LDS and one
// thread per physical page takes their max.
//
// Top-K.  Scores are mapped to order-preserving 64-bit keys held in
// registers; a most significant digit first radix select finds the K-th
// largest key.  The passes start at the highest bit in which the keys differ
// (the bits above it are common to all keys) and take the next 8 bits each;
// the histogram is in LDS, double-buffered so a pass needs two barriers.
// Equal keys are taken in ascending page order (ties to the lower page
// index); an ordered compaction writes the selected pages in ascending order.
// Up to 4096 pages per sequence the ranking runs inside the score kernel: the
// last score workgroup of a (sequence, head) to finish, counted with an
// arrival counter, ranks that head; above that a separate top-K kernel does.
// The page statistics are read once per launch and carry the non-temporal
// hint.
#include "lsa_internal.h"

namespace lsa {
namespace {

template <int EB, int D>
struct ScoreShape {
    static constexpr int C = 16 / EB;        // channels per lane (one 16-byte load)
    static constexpr int LPL = D / C;        // lanes per logical page
    static constexpr int LPP = kWave / LPL;  // logical pages per wavefront pass
};

constexpr int kScoreThreads = 256;
// logical pages per lane group and workgroup, chosen per instance so that
// three wavefronts fit per SIMD (at most 168 VGPRs), which hides one
// wavefront's statistics loads behind another's arithmetic:
// - int4 (a lane holds 16 channels of fp64 query terms): seven pages
//   (config 5: 102 us per score launch at eight pages and two wavefronts per
//   SIMD, 90 at six, 87 at seven);
// - bf16: eleven, fewer and fuller workgroups; 44 physical pages per
//   workgroup put a 1025-page selection of 8 sequences x 4 heads in 768
//   workgroups, one per slot of the chip (config 2: 29.1 us per score launch
//   at eight, 28.4 at ten, 26.8 at eleven);
// - with the 16-pages-per-thread top-K fused in, one page fewer each (one
//   more would cross 168 VGPRs);
// - max aggregation keeps the packed statistics across one pass per query
//   head: bf16 fits three wavefronts per SIMD at six pages (160 VGPRs;
//   config 2: 42.9 us per selection against 46.8 at ten and 45.0 at nine,
//   both at two wavefronts per SIMD); int4 needs over 200 VGPRs at any
//   count and keeps six.
constexpr int score_iters(int kv_dtype, int fused_pt, bool agg_max) {
    if (kv_dtype == LSA_INT4) return agg_max || fused_pt == 16 ? 6 : 7;
    if (kv_dtype == LSA_BF16) return agg_max ? 6 : fused_pt == 16 ? 10 : 11;
    return 8;
}
constexpr int kMaxLogicalPerBlock = 1024;  // LDS slots for logical scores

// Qp / Qn of this lane's channels over the group's query heads h0 .. h1-1, fp64.
template <int C>
__device__ __forceinline__ void load_q_pos_neg(const ScoreArgs &a, int b, int kv, int ch0, int h0, int h1,
                                                double (&qp)[C], double (&qn)[C]) {
    const int G = a.num_q_heads / a.num_kv_heads;
#pragma unroll
    for (int c = 0; c < C; ++c) { qp[c] = 0.0; qn[c] = 0.0; }
    for (int h = h0; h < h1; ++h) {
        const size_t row = ((size_t)b * a.num_q_heads + (size_t)kv * G + h) * a.head_dim + ch0;
        float x[C];
        if (a.q_dtype == LSA_BF16) {
            const uint16_t *p = static_cast<const uint16_t *>(a.q) + row;
#pragma unroll
            for (int c = 0; c < C; c += 8) {
                const uint4 u = *reinterpret_cast<const uint4 *>(p + c);
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 8 && c + e < C; ++e) x[c + e] = (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
            }
        } else {
            const float *p = static_cast<const float *>(a.q) + row;
#pragma unroll
            for (int c = 0; c < C; c += 4) {
                const float4 u = *reinterpret_cast<const float4 *>(p + c);
                x[c] = u.x; x[c + 1] = u.y; x[c + 2] = u.z; x[c + 3] = u.w;
            }
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const double v = (double)x[c];
            qp[c] += fmax(v, 0.0);
            qn[c] += fmin(v, 0.0);
        }
    }
}

// min / max of this lane's C channels over the current logical page's rows
// held by the wavefront (lane group q of the LPP groups takes rows q, q + LPP,
// ...), combined over the groups so every lane ends with all rows.  Float
// channels for f32 / bf16 pools, 4-bit codes (as floats) for int4 pools.
template <int KV_DT, int D, int C, int LPL, int LPP>
__device__ __forceinline__ void current_page_minmax(const ScoreArgs &a, size_t page_base, int row0, int rows, int q,
                                                    int ch0, float (&kmin)[C], float (&kmax)[C]) {
#pragma unroll
    for (int c = 0; c < C; ++c) { kmin[c] = __builtin_inff(); kmax[c] = -__builtin_inff(); }
    constexpr int RB = 4;                       // rows per lane and batch, loaded together
    for (int r0 = 0; r0 < rows; r0 += RB * LPP) {
        if constexpr (KV_DT == LSA_INT4) {
            uint2 u[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const int rr = r0 + q + i * LPP;
                u[i] = rr < rows ? *reinterpret_cast<const uint2 *>(static_cast<const uint8_t *>(a.k) +
                                                                    (page_base + key_offset(row0 + rr, ch0, D)) / 2)
                                 : make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (r0 + q + i * LPP >= rows) continue;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const uint32_t byte = ((c < 8 ? u[i].x : u[i].y) >> (8 * ((c / 2) % 4))) & 0xFFu;
                    const float code = (float)((c & 1) ? (byte >> 4) : (byte & 15u));
                    kmin[c] = fminf(kmin[c], code);
                    kmax[c] = fmaxf(kmax[c], code);
                }
            }
        } else {
            uint4 u[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const int rr = r0 + q + i * LPP;
                u[i] = rr < rows ? *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.k) +
                                                                    (page_base + key_offset(row0 + rr, ch0, D)) *
                                                                        (KV_DT == LSA_F32 ? 4 : 2))
                                 : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (r0 + q + i * LPP >= rows) continue;
                const uint32_t w[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    float x;
                    if constexpr (KV_DT == LSA_BF16) x = (c & 1) ? bf16_hi(w[c / 2]) : bf16_lo(w[c / 2]);
                    else x = __uint_as_float(w[c]);
                    kmin[c] = fminf(kmin[c], x);
                    kmax[c] = fmaxf(kmax[c], x);
                }
            }
        }
    }
    // combine the lane groups that share this lane's channels (the lanes
    // with the same lane % LPL): rotations inside a row of 16, then swaps
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if constexpr (LPL <= 4) {
            kmin[c] = fminf(kmin[c], __uint_as_float(dpp_u<kDppRowRor4>(__float_as_uint(kmin[c]))));
            kmax[c] = fmaxf(kmax[c], __uint_as_float(dpp_u<kDppRowRor4>(__float_as_uint(kmax[c]))));
        }
        if constexpr (LPL <= 8) {
            kmin[c] = fminf(kmin[c], __uint_as_float(dpp_u<kDppRowRor8>(__float_as_uint(kmin[c]))));
            kmax[c] = fmaxf(kmax[c], __uint_as_float(dpp_u<kDppRowRor8>(__float_as_uint(kmax[c]))));
        }
        if constexpr (LPL <= 16) {
            kmin[c] = -max_xor16(-kmin[c]);
            kmax[c] = max_xor16(kmax[c]);
        }
        kmin[c] = -max_xor32(-kmin[c]);
        kmax[c] = max_xor32(kmax[c]);
    }
}

// ---------------------------------------------------------------------------
// top-K of one (sequence, retrieval head): by a 1024-thread workgroup of its
// own, or by the last score workgroup of the head (256 threads)
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kTopkPerThread = 16;        // pages per thread at most: up to 16384 pages

__device__ __forceinline__ unsigned long long order_key(double x) {
    x = x + 0.0;                                  // -0 -> +0
    const unsigned long long u = __double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ void store_agent_d(double *p, double v) {
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), (unsigned long long)__double_as_longlong(v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double load_agent_d(const double *p) {
    return __longlong_as_double((long long)__hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// exclusive prefix sum over the NT threads of a 32-bit packed counter
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wave_tot) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const uint32_t incl = wave_inclusive_scan(v);
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t add = 0;
    for (int w = 0; w < wave; ++w) add += wave_tot[w];
    return incl - v + add;
}

// The K largest of the n = ceil(L / N_P) scores P[0..n) into out, ascending by
// page, ties to the lower page, -1 padded; NT threads, PT pages per thread
// (NT * PT >= max_pages).  AGENT: P was written by other workgroups of this
// launch and is read with agent-scope loads.
template <int NT, int PT, bool AGENT>
__device__ __forceinline__ void topk_rows(const double *P, int L, int page_size, int max_pages, int K,
                                          int32_t *out) {
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t sh_digit, sh_above, sh_done;
    __shared__ uint32_t wave_tot[NT / kWave];
    __shared__ unsigned long long sh_and[NT / kWave], sh_or[NT / kWave];
    const int tid = threadIdx.x;

    // thread t owns the contiguous pages [t*seg, t*seg + cnt); the scores are
    // loaded for every row slot at once, and the entries past the sequence's
    // last page are dropped afterwards
    constexpr int seg = PT;
    const int i0 = min(max_pages, tid * seg);
    double pv[PT];
#pragma unroll
    for (int e = 0; e < PT; ++e) {
        if constexpr (AGENT) pv[e] = i0 + e < max_pages ? load_agent_d(P + i0 + e) : 0.0;
        else pv[e] = i0 + e < max_pages ? P[i0 + e] : 0.0;
    }
    const int n = (L + page_size - 1) / page_size;
    if (n <= K) {                                 // every page, ascending, padded with -1
        for (int i = tid; i < K; i += NT) out[i] = i < n ? i : -1;
        return;
    }
    const int cnt = max(0, min(n, i0 + seg) - i0);
    unsigned long long key[PT];
#pragma unroll
    for (int e = 0; e < PT; ++e) key[e] = e < cnt ? order_key(pv[e]) : 0ull;

    // The bits above the highest one that differs between keys are shared by
    // every key and decide nothing: the radix passes start there, each pass
    // resolving the next (up to) 8 bits of the K-th largest key.
    unsigned long long k_and = ~0ull, k_or = 0ull;
#pragma unroll
    for (int e = 0; e < PT; ++e)
        if (e < cnt) { k_and &= key[e]; k_or |= key[e]; }
    wave_and_or(k_and, k_or);
    if (tid % kWave == 0) { sh_and[tid / kWave] = k_and; sh_or[tid / kWave] = k_or; }
    for (int i = tid; i < 256; i += NT) hist[0][i] = 0;
    __syncthreads();
    k_and = ~0ull; k_or = 0ull;
    for (int w2 = 0; w2 < NT / kWave; ++w2) { k_and &= sh_and[w2]; k_or |= sh_or[w2]; }
    const unsigned long long differ = k_and ^ k_or;      // bits that are not the same in every key
    int hi = differ ? 64 - __clzll((long long)differ) : 0;   // one past the highest differing bit
    unsigned long long mask = hi >= 64 ? 0ull : (~0ull << hi);
    unsigned long long prefix = k_and & mask;
    uint32_t need = (uint32_t)K;
    int buf = 0;
    while (hi > 0) {
        const int lo = max(0, hi - 8);
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
#pragma unroll
        for (int e = 0; e < PT; ++e)
            if (e < cnt && (key[e] & mask) == prefix) atomicAdd(&hist[buf][uint32_t(key[e] >> lo) & dmask], 1u);
        for (int i = tid; i < 256; i += NT) hist[buf ^ 1][i] = 0;    // the next pass's histogram
        __syncthreads();
        if (tid < kWave) {
            // lane l owns bins 4l..4l+3; count the elements in higher bins
            const uint32_t *hb = hist[buf];
            const uint32_t c0 = hb[4 * tid], c1 = hb[4 * tid + 1], c2 = hb[4 * tid + 2], c3 = hb[4 * tid + 3];
            const uint32_t mine = c0 + c1 + c2 + c3;
            const uint32_t incl = wave_inclusive_scan(mine);
            const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
            uint32_t above = total - incl;        // elements in bins of higher lanes
            const uint32_t cs[4] = {c0, c1, c2, c3};
            for (int qd = 3; qd >= 0; --qd) {
                if (above < need && above + cs[qd] >= need) {
                    sh_digit = 4 * tid + qd;
                    sh_above = above;
                    sh_done = above + cs[qd] == need;   // the whole bin is taken
                }
                above += cs[qd];
            }
        }
        __syncthreads();
        need -= sh_above;
        prefix |= (unsigned long long)sh_digit << lo;
        mask |= (unsigned long long)dmask << lo;
        hi = lo;
        if (sh_done) break;
        buf ^= 1;
    }

    // ordered compaction
    uint32_t c = 0;                               // low 16 bits: greater, high 16 bits: equal
#pragma unroll
    for (int e = 0; e < PT; ++e) {
        if (e >= cnt) continue;
        const unsigned long long km = key[e] & mask;
        c += km > prefix ? 1u : (km == prefix ? 0x10000u : 0u);
    }
    const uint32_t excl = block_exclusive_scan<NT>(c, wave_tot);
    uint32_t gt_before = excl & 0xFFFFu;
    uint32_t eq_before = excl >> 16;
#pragma unroll
    for (int e = 0; e < PT; ++e) {
        if (e >= cnt) continue;
        const unsigned long long km = key[e] & mask;
        if (km > prefix) {
            out[gt_before + min(eq_before, need)] = i0 + e;
            ++gt_before;
        } else if (km == prefix) {
            if (eq_before < need) out[gt_before + eq_before] = i0 + e;
            ++eq_before;
        }
    }
}

// PT: pages per thread, the smallest power of two with kTopkThreads * PT >=
// max_pages (every per-page loop is unrolled over PT slots).
template <int PT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
    const int r = blockIdx.x % a.n_ret;
    const int b = blockIdx.x / a.n_ret;
    const int kv = a.ret_heads[r];
    topk_rows<kTopkThreads, PT, false>(a.phys + ((size_t)b * a.num_kv_heads + kv) * a.max_pages, a.seq_lens[b],
                                       a.page_size, a.max_pages, a.k,
                                       a.selected + ((size_t)b * a.num_kv_heads + kv) * a.k);
}

// KV_DT: LSA_F32, LSA_BF16 (stats in that type) or LSA_INT4 (code stats).
// AGG_MAX: the group's heads are scored one by one and their scores combined
// by max; otherwise their sum is formed with one folded (Qp, Qn) pass.
// FPT > 0: the physical scores go out with agent-scope stores and the last
// workgroup of a (sequence, head) to finish runs the head's top-K with FPT
// pages per thread (the hand-off of the decode kernel's split-KV merge).
template <int KV_DT, int D, bool AGG_MAX, int FPT>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreArgs a) {
    constexpr int EB = KV_DT == LSA_F32 ? 4 : (KV_DT == LSA_BF16 ? 2 : 1);
    using S = ScoreShape<EB, D>;
    constexpr int C = S::C, LPL = S::LPL, LPP = S::LPP;
    constexpr int GROUPS = (kScoreThreads / kWave) * LPP;   // lane groups per workgroup
    constexpr int IT = score_iters(KV_DT, FPT, AGG_MAX);
    __shared__ double s_log[kMaxLogicalPerBlock];

    const int blk = blockIdx.x % a.blocks_per_head;
    const int rest = blockIdx.x / a.blocks_per_head;
    const int r = rest % a.n_ret;
    const int b = rest / a.n_ret;
    const int kv = a.ret_heads[r];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int lg = wave * LPP + lane / LPL;       // lane group in the workgroup
    const int ch0 = (lane % LPL) * C;

    const int g = a.page_size / a.logical_page;
    const int m0 = blk * a.pages_per_block;
    const int j0 = m0 * g;
    // page-table entries of this lane group's logical pages, loaded together
    // with seq_lens and q (nothing here waits on another load)
    int pools[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int m = (j0 + lg + it * GROUPS) / g;
        pools[it] = m < a.max_pages ? a.page_table[(size_t)b * a.max_pages + m] : 0;
    }
    const int L = a.seq_lens[b];
    const int G = a.num_q_heads / a.num_kv_heads;
    const int n_pages = (L + a.page_size - 1) / a.page_size;
    if (m0 < n_pages) {                           // (uniform: a workgroup past the last page only arrives)
    const int m1 = min(m0 + a.pages_per_block, n_pages);
    const int nlog = (L + a.logical_page - 1) / a.logical_page;
    const int j1 = min(m1 * g, nlog);
    const int j_cur = (L - 1) / a.logical_page;   // the logical page that holds the current token
    const size_t head_stride = (size_t)g * (KV_DT == LSA_INT4 ? D : 2 * D);

    // every statistics load of the workgroup is issued before any product
    uint4 st_lo[IT], st_hi[IT];
    uint32_t szw[IT];                             // int4: the page's fp16 scale | zero << 16
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int j = j0 + lg + it * GROUPS;
        st_lo[it] = make_uint4(0, 0, 0, 0);
        st_hi[it] = make_uint4(0, 0, 0, 0);
        szw[it] = 0;
        if (j < j1 && j != j_cur) {
            const size_t hp = (size_t)pools[it] * a.num_kv_heads + kv;
            const int jl = j % g;
            if constexpr (KV_DT == LSA_INT4) {
                st_lo[it] = load_stream16(static_cast<const uint8_t *>(a.stats) + hp * head_stride + (size_t)jl * D + ch0);
                szw[it] = load_stream4(a.k_sz + hp * 2);
            } else {
                const char *st = static_cast<const char *>(a.stats) + (hp * head_stride + (size_t)jl * 2 * D + ch0) * EB;
                st_lo[it] = load_stream16(st);
                st_hi[it] = load_stream16(st + (size_t)D * EB);
            }
        }
    }

    // the current logical page's min / max, from its keys, by one whole wavefront
    const bool own_cur = j_cur >= j0 && j_cur < j1 && wave == ((j_cur - j0) % GROUPS) / LPP;
    float cmin[C], cmax[C];
    uint32_t sz_cur = 0;
    if (own_cur) {
        const int pool = a.page_table[(size_t)b * a.max_pages + j_cur / g];
        const size_t hp = (size_t)pool * a.num_kv_heads + kv;
        if constexpr (KV_DT == LSA_INT4) sz_cur = *reinterpret_cast<const uint32_t *>(a.k_sz + hp * 2);
        current_page_minmax<KV_DT, D, C, LPL, LPP>(a, hp * a.page_size * D, (j_cur % g) * a.logical_page,
                                                   L - j_cur * a.logical_page, lane / LPL, ch0, cmin, cmax);
    }

    // int4: S = s * (sum_i Qp c_max + Qn c_min - z * sum_i (Qp + Qn))
    auto finish = [&](double dot, uint32_t sz, double qsum) {
        if constexpr (KV_DT == LSA_INT4)
            return (double)fp16_bits_to_f32(uint16_t(sz)) * (dot - (double)fp16_bits_to_f32(uint16_t(sz >> 16)) * qsum);
        return dot;
    };

    // S^j of every logical page: one pass with the folded group (sum), or one
    // pass per query head combined by max; each slot has its own product chains
    double best[IT], best_cur = 0.0;
    const int n_pass = AGG_MAX ? G : 1;
    for (int hv = 0; hv < n_pass; ++hv) {
        if constexpr (AGG_MAX) {
            // keep the statistics packed across passes: without this the
            // compiler converts every slot to fp64 once, before the loop, which
            // needs four times the registers and leaves one wavefront per SIMD
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                if constexpr (KV_DT == LSA_INT4)
                    asm volatile("" : "+v"(st_lo[it].x), "+v"(st_lo[it].y), "+v"(st_lo[it].z), "+v"(st_lo[it].w),
                                 "+v"(szw[it]));
                else
                    asm volatile("" : "+v"(st_lo[it].x), "+v"(st_lo[it].y), "+v"(st_lo[it].z), "+v"(st_lo[it].w),
                                 "+v"(st_hi[it].x), "+v"(st_hi[it].y), "+v"(st_hi[it].z), "+v"(st_hi[it].w));
            }
        }
        double qp[C], qn[C];
        load_q_pos_neg<C>(a, b, kv, ch0, AGG_MAX ? hv : 0, AGG_MAX ? hv + 1 : G, qp, qn);
        double qsum = 0.0;                        // int4 only: sum over all channels of Qp + Qn
        if constexpr (KV_DT == LSA_INT4) {
#pragma unroll
            for (int c = 0; c < C; ++c) qsum += qp[c] + qn[c];
            qsum = group_sum_d<LPL>(qsum);
        }
        if (own_cur) {
            double c0 = 0.0, c1 = 0.0;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                c0 = fma(qp[c], (double)cmax[c], c0);
                c1 = fma(qn[c], (double)cmin[c], c1);
            }
            const double sj = finish(group_sum_d<LPL>(c0 + c1), sz_cur, qsum);
            best_cur = hv == 0 ? sj : fmax(best_cur, sj);
        }
        double acc[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            double c0 = 0.0, c1 = 0.0;
            if constexpr (KV_DT == LSA_INT4) {
                const uint32_t wd[4] = {st_lo[it].x, st_lo[it].y, st_lo[it].z, st_lo[it].w};
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const uint32_t byte = (wd[c / 4] >> (8 * (c % 4))) & 0xFFu;
                    c0 = fma(qp[c], (double)(byte >> 4), c0);
                    c1 = fma(qn[c], (double)(byte & 15u), c1);
                }
            } else {
                const uint32_t wl[4] = {st_lo[it].x, st_lo[it].y, st_lo[it].z, st_lo[it].w};
                const uint32_t wh[4] = {st_hi[it].x, st_hi[it].y, st_hi[it].z, st_hi[it].w};
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    float kmin, kmax;
                    if constexpr (KV_DT == LSA_BF16) {
                        kmin = (c & 1) ? bf16_hi(wl[c / 2]) : bf16_lo(wl[c / 2]);
                        kmax = (c & 1) ? bf16_hi(wh[c / 2]) : bf16_lo(wh[c / 2]);
                    } else {
                        kmin = __uint_as_float(wl[c]);
                        kmax = __uint_as_float(wh[c]);
                    }
                    c0 = fma(qp[c], (double)kmax, c0);
                    c1 = fma(qn[c], (double)kmin, c1);
                }
            }
            acc[it] = c0 + c1;
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const double sj = finish(group_sum_d<LPL>(acc[it]), szw[it], qsum);
            best[it] = hv == 0 ? sj : fmax(best[it], sj);
        }
    }
    if (own_cur && lane == 0) s_log[j_cur - j0] = best_cur;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int j = j0 + lg + it * GROUPS;
        if (j < j1 && j != j_cur && lane % LPL == 0) s_log[j - j0] = best[it];
    }
    __syncthreads();
    // P_m = max over the logical pages of physical page m
    for (int m = m0 + threadIdx.x; m < m1; m += blockDim.x) {
        const int ja = m * g - j0, jb = min((m + 1) * g, j1) - j0;
        double best = s_log[ja];
        for (int jj = ja + 1; jj < jb; ++jj) best = fmax(best, s_log[jj]);
        double *dst = a.phys + ((size_t)b * a.num_kv_heads + kv) * a.max_pages + m;
        if constexpr (FPT > 0) store_agent_d(dst, best + 0.0);
        else *dst = best + 0.0;
    }
    }
    if constexpr (FPT > 0) {
        __shared__ int s_last;
        // this wavefront's score stores have reached the coherence point
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) {
            int32_t *cnt = a.counters + (size_t)b * a.num_kv_heads + kv;
            const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int last = old == a.blocks_per_head - 1;
            if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = last;
        }
        __syncthreads();
        if (s_last)
            topk_rows<kScoreThreads, (FPT > 0 ? FPT : 1), true>(
                a.phys + ((size_t)b * a.num_kv_heads + kv) * a.max_pages, L, a.page_size, a.max_pages, a.k_pages,
                a.selected + ((size_t)b * a.num_kv_heads + kv) * a.k_pages);
    }
}

template <int KV_DT, bool AGG_MAX, int FPT>
void launch_score_fpt(const ScoreArgs &a, unsigned grid, hipStream_t s) {
    if (a.head_dim == 128) hipLaunchKernelGGL((score_kernel<KV_DT, 128, AGG_MAX, FPT>), dim3(grid), dim3(kScoreThreads), 0, s, a);
    else hipLaunchKernelGGL((score_kernel<KV_DT, 64, AGG_MAX, FPT>), dim3(grid), dim3(kScoreThreads), 0, s, a);
}

template <int KV_DT, bool AGG_MAX>
hipError_t launch_score_agg(const ScoreArgs &a, unsigned grid, hipStream_t s) {
    switch (a.fused_pt) {
        case 0: launch_score_fpt<KV_DT, AGG_MAX, 0>(a, grid, s); break;
        case 4: launch_score_fpt<KV_DT, AGG_MAX, 4>(a, grid, s); break;
        case 8: launch_score_fpt<KV_DT, AGG_MAX, 8>(a, grid, s); break;
        case 16: launch_score_fpt<KV_DT, AGG_MAX, 16>(a, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int KV_DT>
hipError_t launch_score_dt(const ScoreArgs &a, unsigned grid, hipStream_t s) {
    return a.aggregation == LSA_AGG_MAX ? launch_score_agg<KV_DT, true>(a, grid, s)
                                        : launch_score_agg<KV_DT, false>(a, grid, s);
}

}  // namespace

int score_pages_per_block(int kv_dtype, int head_dim, int page_size, int logical_page, int fused_pt, bool agg_max) {
    // lane groups per workgroup x iterations, in logical pages, over g
    const int eb = kv_dtype == LSA_F32 ? 4 : (kv_dtype == LSA_BF16 ? 2 : 1);
    const int lpl = head_dim / (16 / eb);
    const int groups = (kScoreThreads / kWave) * (kWave / lpl);
    const int g = page_size / logical_page;
    int ppb = groups * score_iters(kv_dtype, fused_pt, agg_max) / g;
    ppb = ppb < 1 ? 1 : ppb;
    return ppb * g > kMaxLogicalPerBlock ? kMaxLogicalPerBlock / g : ppb;
}

int topk_max_pages() { return kTopkThreads * kTopkPerThread; }

int score_fused_pt(int max_pages) {
    const int per = (max_pages + kScoreThreads - 1) / kScoreThreads;
    return per <= 4 ? 4 : per <= 8 ? 8 : per <= 16 ? 16 : 0;
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t s) {
    const long long grid = (long long)a.batch * a.n_ret * a.blocks_per_head;
    if (grid == 0) return hipSuccess;
    if (a.kv_dtype == LSA_INT4) return launch_score_dt<LSA_INT4>(a, (unsigned)grid, s);
    if (a.kv_dtype == LSA_BF16) return launch_score_dt<LSA_BF16>(a, (unsigned)grid, s);
    return launch_score_dt<LSA_F32>(a, (unsigned)grid, s);
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t s) {
    const long long grid = (long long)a.batch * a.n_ret;
    if (grid == 0) return hipSuccess;
    const int per = (a.max_pages + kTopkThreads - 1) / kTopkThreads;
    const dim3 g((unsigned)grid), blk(kTopkThreads);
    if (per <= 1) hipLaunchKernelGGL(topk_kernel<1>, g, blk, 0, s, a);
    else if (per <= 2) hipLaunchKernelGGL(topk_kernel<2>, g, blk, 0, s, a);
    else if (per <= 4) hipLaunchKernelGGL(topk_kernel<4>, g, blk, 0, s, a);
    else if (per <= 8) hipLaunchKernelGGL(topk_kernel<8>, g, blk, 0, s, a);
    else hipLaunchKernelGGL(topk_kernel<kTopkPerThread>, g, blk, 0, s, a);
    return hipGetLastError();
}

}  // namespace lsa
