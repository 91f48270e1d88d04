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
// Top-K.  The scores stay in registers; the K-th largest is found by value
// (linear bins between the smallest and largest score still in question,
// then one wavefront ranking the few scores that share the bin of the K-th;
// see topk_rows).  Equal scores are taken in ascending page order (ties to
// the lower page index); an ordered compaction writes the selected pages in
// ascending order.
// Up to 4096 pages per sequence the ranking runs inside the score kernel: the
// last score workgroup of a (sequence, head) to finish, counted with an
// arrival counter, ranks that head; above that a separate top-K kernel does.
// The page statistics are read once per launch and carry the non-temporal
// hint.
#include "lsa_internal.h"

namespace lsa {
namespace {

typedef int int32x4 __attribute__((ext_vector_type(4)));

// sum of v over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four k-groups of a
// 16 x 16 MFMA tile column), in every lane
__device__ __forceinline__ double sum_kgroups_d(double v) {
    uint32_t l0, l1, h0, h1;
    unsigned long long u = __double_as_longlong(v);
    pair16((uint32_t)u, l0, l1);
    pair16((uint32_t)(u >> 32), h0, h1);
    v = __longlong_as_double((long long)(((unsigned long long)h0 << 32) | l0)) +
        __longlong_as_double((long long)(((unsigned long long)h1 << 32) | l1));
    u = __double_as_longlong(v);
    pair32((uint32_t)u, l0, l1);
    pair32((uint32_t)(u >> 32), h0, h1);
    return __longlong_as_double((long long)(((unsigned long long)h0 << 32) | l0)) +
           __longlong_as_double((long long)(((unsigned long long)h1 << 32) | l1));
}

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
//   (16 sequences x 4 heads at 256K tokens: 102 us per score launch at eight
//   pages and two wavefronts per SIMD, 90 at six, 87 at seven);
// - bf16: eleven, fewer and fuller workgroups; 44 physical pages per
//   workgroup put a 1025-page selection of 8 sequences x 4 heads in 768
//   workgroups, one per slot of the chip (29.1 us per score launch at
//   eight, 28.4 at ten, 26.8 at eleven);
// - with the 16-pages-per-thread top-K fused in, one page fewer each (one
//   more would cross 168 VGPRs);
// - max aggregation keeps the packed statistics across one pass per query
//   head: bf16 fits three wavefronts per SIMD at six pages (160 VGPRs; 8
//   sequences x 4 heads at 64K tokens: 42.9 us per selection against 46.8
//   at ten and 45.0 at nine, both at two wavefronts per SIMD); int4 needs
//   over 200 VGPRs at any count and keeps six.
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
                                                    int ch0, const void *knew_row, float (&kmin)[C], float (&kmax)[C]) {
#pragma unroll
    for (int c = 0; c < C; ++c) { kmin[c] = __builtin_inff(); kmax[c] = -__builtin_inff(); }
    const int bs = block_shift(a.page_size);
    constexpr int RB = 4;                       // rows per lane and batch, loaded together
    for (int r0 = 0; r0 < rows; r0 += RB * LPP) {
        if constexpr (KV_DT == LSA_INT4) {
            uint2 u[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const int rr = r0 + q + i * LPP;
                const uint8_t *src = knew_row && rr == rows - 1
                                         ? static_cast<const uint8_t *>(knew_row) + ch0 / 2
                                         : static_cast<const uint8_t *>(a.k) + (page_base + key_offset(row0 + rr, ch0, D, bs)) / 2;
                u[i] = rr < rows ? *reinterpret_cast<const uint2 *>(src) : make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
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
                constexpr int EBk = KV_DT == LSA_F32 ? 4 : 2;
                const char *src = knew_row && rr == rows - 1
                                      ? static_cast<const char *>(knew_row) + (size_t)ch0 * EBk
                                      : static_cast<const char *>(a.k) + (page_base + key_offset(row0 + rr, ch0, D, bs)) * EBk;
                u[i] = rr < rows ? *reinterpret_cast<const uint4 *>(src) : make_uint4(0, 0, 0, 0);
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

// min and max of doubles over the wavefront (every lane gets both)
__device__ __forceinline__ void wave_minmax_d(double &lo, double &hi) {
    lo = fmin(lo, dpp_d<kDppQuadSwap1>(lo)); hi = fmax(hi, dpp_d<kDppQuadSwap1>(hi));
    lo = fmin(lo, dpp_d<kDppQuadSwap2>(lo)); hi = fmax(hi, dpp_d<kDppQuadSwap2>(hi));
    lo = fmin(lo, dpp_d<kDppHalfMirror>(lo)); hi = fmax(hi, dpp_d<kDppHalfMirror>(hi));
    lo = fmin(lo, dpp_d<kDppMirror>(lo)); hi = fmax(hi, dpp_d<kDppMirror>(hi));
    auto both = [](double v, bool x32, double &p, double &q) {
        const unsigned long long u = __double_as_longlong(v);
        uint32_t l0, l1, h0, h1;
        if (x32) { pair32((uint32_t)u, l0, l1); pair32((uint32_t)(u >> 32), h0, h1); }
        else { pair16((uint32_t)u, l0, l1); pair16((uint32_t)(u >> 32), h0, h1); }
        p = __longlong_as_double((long long)(((unsigned long long)h0 << 32) | l0));
        q = __longlong_as_double((long long)(((unsigned long long)h1 << 32) | l1));
    };
    double p, q;
    both(lo, false, p, q); lo = fmin(p, q);
    both(hi, false, p, q); hi = fmax(p, q);
    both(lo, true, p, q); lo = fmin(p, q);
    both(hi, true, p, q); hi = fmax(p, q);
}

// The K largest of the n = ceil(L / N_P) scores P[0..n) into out, ascending by
// page, ties to the lower page, -1 padded; NT threads, PT pages per thread
// (NT * PT >= max_pages - 1).  AGENT: P was written by other workgroups of
// this launch and is read with agent-scope loads.
//
// The threshold T, the K-th largest score, is found by value: the scores
// still in question are binned linearly between their minimum and maximum
// (a monotone map, so a bin holds a contiguous range of values and equal
// scores share a bin), the bin that holds the K-th largest is found from the
// histogram, and the scores outside it are settled.  When at most
// kTopkCand scores share that bin, one wavefront ranks them against each
// other and T is exact; otherwise the bin is binned again.  Linear bins
// spread a smooth distribution of scores over the histogram, so few threads
// meet on one counter.  Pages with scores above T are taken, and of the
// pages scoring exactly T the lowest ones, K in all, in one ordered
// compaction.
// One page past the NT * PT the threads hold (n = NT * PT + 1, which the
// host allows in the score kernel with the group's scores summed at 4 or 8
// pages per thread, and in the separate top-K kernel) is ranked apart: it is
// the last page, n - 1, the highest index, so it loses every tie.  The K
// largest of the others are found as above; the last page joins them exactly
// when its score is above their K-th largest T, and the lowest-ranked of them
// (score T, the highest such page taken) then leaves.
constexpr int kTopkBins = 1024;
constexpr int kTopkCand = 16;

template <int NT, int PT, bool AGENT>
__device__ __forceinline__ void topk_rows(const double *P, int L, int page_size, int max_pages, int K,
                                          int32_t *out) {
    static_assert(PT <= 32, "pages per thread");
    constexpr int NW = NT / kWave;
    __shared__ uint32_t hist[kTopkBins];
    __shared__ double sh_lo[NW], sh_hi[NW];
    __shared__ double cand[kTopkCand];
    __shared__ uint32_t sh_bin, sh_above, sh_ncand, sh_gt;
    __shared__ double sh_T;
    __shared__ uint32_t wave_tot[NW];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

    // thread t owns the contiguous pages [t*seg, t*seg + cnt) of the ns held
    // in registers, seg = ceil(ns / NT) <= PT; their scores are loaded together
    const int n = (L + page_size - 1) / page_size;
    if (n <= K) {                                 // every page, ascending, padded with -1
        for (int i = tid; i < K; i += NT) out[i] = i < n ? i : -1;
        return;
    }
    const bool extra = n > NT * PT;               // (then n == NT * PT + 1: the host's bound)
    const int ns = extra ? n - 1 : n;
    const int seg = (ns + NT - 1) / NT;
    const int i0 = min(ns, tid * seg);
    const int cnt = min(ns, i0 + seg) - i0;
    double sc[PT];
#pragma unroll
    for (int e = 0; e < PT; ++e) {
        double v = 0.0;
        if (e < cnt) v = AGENT ? load_agent_d(P + i0 + e) : P[i0 + e];
        sc[e] = v + 0.0;                          // -0 -> +0
    }
    double x_last = 0.0;                          // the score of page n - 1 when it is ranked apart
    if (extra) x_last = (AGENT ? load_agent_d(P + n - 1) : P[n - 1]) + 0.0;
    uint32_t act = cnt >= 32 ? ~0u : (1u << cnt) - 1u;   // pages still in question
    uint32_t need = (uint32_t)K;                  // how many of them are taken
    double T;
    uint32_t need_eq;                             // pages scoring exactly T that are taken
    for (;;) {
        double lo = __builtin_inf(), hi = -__builtin_inf();
#pragma unroll
        for (int e = 0; e < PT; ++e)
            if ((act >> e) & 1u) { lo = fmin(lo, sc[e]); hi = fmax(hi, sc[e]); }
        wave_minmax_d(lo, hi);
        if (lane == 0) { sh_lo[wave] = lo; sh_hi[wave] = hi; }
        for (int i = tid; i < kTopkBins; i += NT) hist[i] = 0;
        if (tid == 0) sh_ncand = 0;
        __syncthreads();
        lo = sh_lo[0];
        hi = sh_hi[0];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) { lo = fmin(lo, sh_lo[w2]); hi = fmax(hi, sh_hi[w2]); }
        if (!(hi > lo)) { T = hi; need_eq = need; break; }     // every score in question is equal
        const double scale = (double)kTopkBins / (hi - lo);
        // (scale may overflow for a range of a few denormals: then lo -> 0, the rest -> last)
        auto bin_of = [&](double x) {
            const double f = x == lo ? 0.0 : (x - lo) * scale;
            return f < (double)(kTopkBins - 1) ? (int)f : kTopkBins - 1;
        };
#pragma unroll
        for (int e = 0; e < PT; ++e)
            if ((act >> e) & 1u) atomicAdd(&hist[bin_of(sc[e])], 1u);
        __syncthreads();
        if (wave == 0) {
            // lane l owns bins 16 l .. 16 l + 15; count the scores in higher bins
            constexpr int BPL = kTopkBins / kWave;
            const uint4 *hl = reinterpret_cast<const uint4 *>(hist + BPL * lane);
            uint32_t mine = 0;
#pragma unroll
            for (int q = 0; q < BPL / 4; ++q) {
                const uint4 h4 = hl[q];
                mine += h4.x + h4.y + h4.z + h4.w;
            }
            const uint32_t incl = wave_inclusive_scan(mine);
            const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
            uint32_t above = total - incl;        // scores in the bins of higher lanes
            if (above < need && above + mine >= need) {   // (one lane) the bin is among mine
#pragma unroll
                for (int q = BPL - 1; q >= 0; --q) {
                    const uint32_t cq = hist[BPL * lane + q];
                    if (above < need && above + cq >= need) { sh_bin = BPL * lane + q; sh_above = above; }
                    above += cq;
                }
            }
        }
        __syncthreads();
        const int bstar = (int)sh_bin;
        need -= sh_above;
        const uint32_t m = hist[bstar];           // scores in the bin that holds T
#pragma unroll
        for (int e = 0; e < PT; ++e)
            if (((act >> e) & 1u) && bin_of(sc[e]) != bstar) act &= ~(1u << e);
        if (m <= (uint32_t)kTopkCand) {
#pragma unroll
            for (int e = 0; e < PT; ++e)
                if ((act >> e) & 1u) cand[atomicAdd(&sh_ncand, 1u)] = sc[e];
            __syncthreads();
            if (wave == 0) {
                // T is the candidate x with (greater) < need <= (greater or equal)
                const double x = lane < (int)m ? cand[lane] : 0.0;
                uint32_t gt = 0, ge = 0;
                for (uint32_t j = 0; j < m; ++j) {
                    const double y = cand[j];
                    gt += y > x;
                    ge += y >= x;
                }
                if (lane < (int)m && gt < need && need <= ge) { sh_T = x; sh_gt = gt; }
            }
            __syncthreads();
            T = sh_T;
            need_eq = need - sh_gt;
            break;
        }
        __syncthreads();                          // (every thread has read hist[bstar])
    }

    // the last page ranked apart joins when it beats T; one page scoring T leaves
    // (need_eq >= 1: T is the K-th largest of the others)
    const bool take_last = extra && x_last > T;
    if (take_last) --need_eq;

    // ordered compaction
    uint32_t c = 0;                               // low 16 bits: greater, high 16 bits: equal
#pragma unroll
    for (int e = 0; e < PT; ++e)
        if (e < cnt) c += sc[e] > T ? 1u : (sc[e] == T ? 0x10000u : 0u);
    const uint32_t excl = block_exclusive_scan<NT>(c, wave_tot);
    uint32_t gt_before = excl & 0xFFFFu;
    uint32_t eq_before = excl >> 16;
#pragma unroll
    for (int e = 0; e < PT; ++e) {
        if (e >= cnt) continue;
        if (sc[e] > T) {
            out[gt_before + min(eq_before, need_eq)] = i0 + e;
            ++gt_before;
        } else if (sc[e] == T) {
            if (eq_before < need_eq) out[gt_before + eq_before] = i0 + e;
            ++eq_before;
        }
    }
    if (take_last && tid == 0) out[K - 1] = n - 1;   // the highest page index: the last slot
}

// NT threads, PT pages per thread: the smallest power of two with NT * PT >=
// max_pages - 1 (every per-page loop is unrolled over PT slots; a last page
// past NT * PT is ranked apart).  The 4097 pages of a 256K-token sequence
// plus its window then rank at 4 per thread (16 sequences x 4 heads, int4
// statistics: 38.4-38.8 us per selection call against 39.3-39.5 at 8 per
// thread; 256 threads at 16 per thread took 41.5-42.1 us).
template <int NT, int PT>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
    const int r = blockIdx.x % a.n_ret;
    const int b = blockIdx.x / a.n_ret;
    const int kv = retrieval_head(a.hm, r);
    topk_rows<NT, PT, false>(a.phys + ((size_t)b * a.num_kv_heads + kv) * a.max_pages, a.seq_lens[b], a.page_size,
                             a.max_pages, a.k, a.selected + ((size_t)b * a.num_kv_heads + kv) * a.k);
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
    const int kv = retrieval_head(a.hm, r);
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
            const size_t hp = (size_t)pools[it] * a.hm.pool_heads + pool_slot(a.hm, kv);
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
        const size_t hp = (size_t)pool * a.hm.pool_heads + pool_slot(a.hm, kv);
        if constexpr (KV_DT == LSA_INT4)     // (t's page may not have its pair in memory yet)
            sz_cur = *reinterpret_cast<const uint32_t *>(a.k_new ? a.k_new_sz + ((size_t)b * a.num_kv_heads + kv) * 2
                                                                  : a.k_sz + hp * 2);
        const void *knew_row = a.k_new ? static_cast<const char *>(a.k_new) +
                                             ((size_t)b * a.num_kv_heads + kv) * D * EB / (KV_DT == LSA_INT4 ? 2 : 1)
                                       : nullptr;
        current_page_minmax<KV_DT, D, C, LPL, LPP>(a, hp * a.page_size * D, (j_cur % g) * a.logical_page,
                                                   L - j_cur * a.logical_page, lane / LPL, ch0, knew_row, cmin, cmax);
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

// ---------------------------------------------------------------------------
// Scoring with the group's scores summed, as a loop with a ring of loads.  A
// workgroup covers pages_per_block physical pages of one (sequence, retrieval
// head), several workgroups per head so that a fixed number run on every CU
// (score_loop_wgs_per_cu).  The pool ids of the range are staged in LDS
// first; each lane group then walks its logical pages j0 + lg, j0 + lg +
// GROUPS, ... through a ring of score_ring register slots: the statistics of
// the (k + ring)-th page are requested as the k-th is scored, so a
// workgroup's memory stream does not drain between pages.  Every slot is
// always loaded (a slot past the range reads the range's first page and is
// discarded), so the wait before a slot counts exactly the loads issued after
// it.  The depth is what keeps HBM busy and no more: every request beyond
// that only lengthens the memory queues, and the loads that start a
// workgroup (its page ids, its queries) then wait behind the other
// workgroups' streams.  Measured on MI355X (selection call, 8 x 4 heads at
// 64K tokens, 67 MB of bf16 statistics): a ring of 2 at two workgroups per
// CU takes 23.5 us, a ring of 8 at four per CU 29.1 us.  int4 statistics
// (16 bytes per lane and page instead of 32, and more arithmetic per byte)
// keep a ring of 8 at four per CU (60 us against 72 us for 16 x 4 heads at
// 256K tokens).
// ---------------------------------------------------------------------------
template <int KV_DT>
__host__ __device__ constexpr int score_ring() { return KV_DT == LSA_INT4 ? 4 : 2; }
constexpr int kMaxRing = 8;
constexpr int kScoreTiles = 4;            // int4 MFMA scoring: 16-page tiles in flight per wavefront
constexpr int kMaxRangePages = 1024;      // physical pages per workgroup (pool ids in LDS)
constexpr int kMaxRangeLogical = 2048;    // logical pages per workgroup (scores in LDS)

template <int KV_DT, int D, int FPT>
__global__ __launch_bounds__(kScoreThreads, 3) void score_loop_kernel(ScoreArgs a) {
    constexpr int EB = KV_DT == LSA_F32 ? 4 : (KV_DT == LSA_BF16 ? 2 : 1);
    using S = ScoreShape<EB, D>;
    constexpr int C = S::C, LPL = S::LPL, LPP = S::LPP;
    constexpr int GROUPS = (kScoreThreads / kWave) * LPP;   // lane groups per workgroup
    // logical scores, then one slot per lane that stores a score no page keeps
    __shared__ double s_log[kMaxRangeLogical + kWave];
    __shared__ unsigned long long s_hp[kMaxRangePages];   // (pool page, head) unit of each page of the range

    const int blk = blockIdx.x % a.blocks_per_head;
    const int rest = blockIdx.x / a.blocks_per_head;
    const int r = rest % a.n_ret;
    const int b = rest / a.n_ret;
    const int kv = retrieval_head(a.hm, r);
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // (a scalar: uniform loops)
    const int lg = wave * LPP + lane / LPL;       // lane group in the workgroup
    const int ch0 = (lane % LPL) * C;

    const int g = a.page_size / a.logical_page;
    const int m0 = blk * a.pages_per_block;       // < max_pages
    const int j0 = m0 * g;
    const int G = a.num_q_heads / a.num_kv_heads;
    const size_t slot_kv = pool_slot(a.hm, kv);
    // seq_lens, the page-table entries of the workgroup's whole range (the
    // row holds max_pages entries; those past the sequence go unused) and,
    // for bf16 / f32 pools, the query are loaded together: one round trip
    // before the ring instead of two
    const int L = a.seq_lens[b];
    const int m_cap = min(a.pages_per_block, a.max_pages - m0);
    for (int i = threadIdx.x; i < m_cap; i += kScoreThreads)
        s_hp[i] = (unsigned long long)a.page_table[(size_t)b * a.max_pages + m0 + i] * a.hm.pool_heads + slot_kv;
    double qp[C], qn[C];                          // Qp, Qn of this lane's channels ch0 ..
    if constexpr (KV_DT != LSA_INT4) load_q_pos_neg<C>(a, b, kv, ch0, 0, G, qp, qn);
    const int n_pages = (L + a.page_size - 1) / a.page_size;
    if (m0 < n_pages) {                           // (uniform: a workgroup past the last page only arrives)
    const int m1 = min(m0 + a.pages_per_block, n_pages);
    const int nlog = (L + a.logical_page - 1) / a.logical_page;
    const int j1 = min(m1 * g, nlog);
    const int j_cur = (L - 1) / a.logical_page;   // the logical page that holds the current token
    // g, the statistics of one (page, head) unit (g * D bytes for int4, g * 2D
    // elements otherwise) and the row of a logical page are powers of two:
    // addresses are shifts
    const int gs = __builtin_ctz(g);
    const int unit_shift = gs + __builtin_ctz(D) + (KV_DT == LSA_INT4 ? 0 : 1 + __builtin_ctz(EB));
    const int row_shift = __builtin_ctz(D) + (KV_DT == LSA_INT4 ? 0 : 1 + __builtin_ctz(EB));

    double qsum = 0.0;                            // int4 only: sum over all channels of Qp + Qn
    // int4: whether every Qp and -Qn term is an integer below 2^32 on the grid
    // 2^lo (bf16 queries of ordinary range span about 21 bits); s_qint then
    // holds those integers (Qp of channel c at c, -Qn at D + c)
    bool on_grid = false;
    int lo = 0;
    __shared__ uint32_t s_qint[2 * 128];
    if constexpr (KV_DT != LSA_INT4) {
        __syncthreads();
    } else {
        // thread t forms one term once for the workgroup: side t / D (0: Qp,
        // 1: -Qn) of channel t % D, with the exponents of its lowest and its
        // leading set bit
        __shared__ int s_lh[2][kScoreThreads / kWave];
        __shared__ double s_qs[kScoreThreads / kWave];
        double v = 0.0;
        if (threadIdx.x < 2 * D) {
            const int side = threadIdx.x / D, c = threadIdx.x % D;
            for (int h = 0; h < G; ++h) {
                const size_t i = ((size_t)b * a.num_q_heads + (size_t)kv * G + h) * D + c;
                const double x = a.q_dtype == LSA_BF16 ? (double)bf16_to_f32(static_cast<const uint16_t *>(a.q)[i])
                                                      : (double)static_cast<const float *>(a.q)[i];
                v += side ? fmax(-x, 0.0) : fmax(x, 0.0);
            }
        }
        int lo_t = 0x7FFFFFFF, hi_t = -0x7FFFFFFF;
        if (v != 0.0) {
            const unsigned long long u = (unsigned long long)__double_as_longlong(v);
            const int ex = int((u >> 52) & 0x7FFu);
            const unsigned long long m = (u & 0xFFFFFFFFFFFFFull) | (1ull << 52);
            lo_t = ex - 1075 + __builtin_ctzll(m);        // exponent of the lowest set bit
            hi_t = ex - 1023;                             // exponent of the leading bit
        }
        lo_t = group_minmax_i<16, false>(lo_t);
        hi_t = group_minmax_i<16, true>(hi_t);
        {
            uint32_t x0, x1;
            pair16((uint32_t)lo_t, x0, x1); lo_t = min((int)x0, (int)x1);
            pair32((uint32_t)lo_t, x0, x1); lo_t = min((int)x0, (int)x1);
            pair16((uint32_t)hi_t, x0, x1); hi_t = max((int)x0, (int)x1);
            pair32((uint32_t)hi_t, x0, x1); hi_t = max((int)x0, (int)x1);
        }
        // the terms' sum over both sides: Qp + Qn = Qp - (-Qn); exact when on_grid
        double vs = group_sum_d<32>(threadIdx.x / D ? -v : v);
        {
            const unsigned long long u = __double_as_longlong(vs);
            uint32_t l0, l1, h0, h1;
            pair32((uint32_t)u, l0, l1);
            pair32((uint32_t)(u >> 32), h0, h1);
            vs = __longlong_as_double((long long)(((unsigned long long)h0 << 32) | l0)) +
                 __longlong_as_double((long long)(((unsigned long long)h1 << 32) | l1));
        }
        if (lane == 0) { s_lh[0][wave] = lo_t; s_lh[1][wave] = hi_t; s_qs[wave] = vs; }
        __syncthreads();
        lo = s_lh[0][0];
        int hi = s_lh[1][0];
        double qs = s_qs[0];
#pragma unroll
        for (int w2 = 1; w2 < kScoreThreads / kWave; ++w2) {
            lo = min(lo, s_lh[0][w2]);
            hi = max(hi, s_lh[1][w2]);
            qs += s_qs[w2];
        }
        if (lo > hi) lo = hi = 0;                 // every term is zero
        on_grid = hi - lo < 32;
        if (on_grid) {
            qsum = qs;
            if (threadIdx.x < 2 * D) s_qint[threadIdx.x] = (uint32_t)ldexp(v, -lo);
        } else {
            // (rare) the fp64 path: this lane's channels, the sum in their order
            load_q_pos_neg<C>(a, b, kv, ch0, 0, G, qp, qn);
#pragma unroll
            for (int c = 0; c < C; ++c) qsum += qp[c] + qn[c];
            qsum = group_sum_d<LPL>(qsum);
        }
        __syncthreads();
    }

    // int4: S = s * (sum_i Qp c_max + Qn c_min - z * sum_i (Qp + Qn))
    auto finish = [&](double dot, uint32_t sz) {
        if constexpr (KV_DT == LSA_INT4)
            return (double)fp16_bits_to_f32(uint16_t(sz)) * (dot - (double)fp16_bits_to_f32(uint16_t(sz >> 16)) * qsum);
        return dot;
    };

    // the current logical page, from its keys, by the wavefront whose lane
    // groups would hold it
    if (j_cur >= j0 && j_cur < j1 && wave == ((j_cur - j0) % GROUPS) / LPP) {
        if constexpr (KV_DT == LSA_INT4)
            if (on_grid) load_q_pos_neg<C>(a, b, kv, ch0, 0, G, qp, qn);
        float cmin[C], cmax[C];
        const size_t hp = s_hp[(j_cur >> gs) - m0];
        uint32_t sz_cur = 0;
        if constexpr (KV_DT == LSA_INT4)     // (t's page may not have its pair in memory yet)
            sz_cur = *reinterpret_cast<const uint32_t *>(a.k_new ? a.k_new_sz + ((size_t)b * a.num_kv_heads + kv) * 2
                                                                  : a.k_sz + hp * 2);
        const void *knew_row = a.k_new ? static_cast<const char *>(a.k_new) +
                                             ((size_t)b * a.num_kv_heads + kv) * D * EB / (KV_DT == LSA_INT4 ? 2 : 1)
                                       : nullptr;
        current_page_minmax<KV_DT, D, C, LPL, LPP>(a, hp * a.page_size * D, (j_cur % g) * a.logical_page,
                                                   L - j_cur * a.logical_page, lane / LPL, ch0, knew_row, cmin, cmax);
        double c0 = 0.0, c1 = 0.0;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            c0 = fma(qp[c], (double)cmax[c], c0);
            c1 = fma(qn[c], (double)cmin[c], c1);
        }
        const double sj = finish(group_sum_d<LPL>(c0 + c1), sz_cur);
        if (lane == 0) s_log[j_cur - j0] = sj;
    }

    // the ring over this lane group's logical pages; the trip count is the
    // wavefront's largest (its first lane group's), the rest is discarded
    const int K_w = max(0, (j1 - j0 - wave * LPP + GROUPS - 1) / GROUPS);
    constexpr int kRing = score_ring<KV_DT>();
    static_assert(kRing <= kMaxRing, "ring");
    uint4 rl[kRing], rh[kRing];
    uint32_t rs[kRing];
    auto issue = [&](int s, int k) {
        int j = j0 + lg + k * GROUPS;
        if (j >= j1) j = j0;                      // past the range: any page of it, discarded
        const unsigned long long hp = s_hp[(j >> gs) - m0];
        const char *st = static_cast<const char *>(a.stats) + (hp << unit_shift) +
                         (((j & (g - 1)) << row_shift) + ch0 * EB);
        rl[s] = load_stream16(st);
        if constexpr (KV_DT == LSA_INT4) rs[s] = load_stream4(a.k_sz + hp * 2);
        else rh[s] = load_stream16(st + D * EB);
        // issue the slot's loads here, in ring order: the wait before a slot then
        // counts exactly the loads of the slots after it
        __builtin_amdgcn_sched_barrier(0);
    };
    // the score of the logical page in ring slot s, from fp64 products
    auto fp_slot = [&](int s) __attribute__((always_inline)) -> double {
            double c0 = 0.0, c1 = 0.0;
            if constexpr (KV_DT == LSA_INT4) {
                // four independent product chains (even / odd channels)
                const uint32_t wd[4] = {rl[s].x, rl[s].y, rl[s].z, rl[s].w};
                double c2 = 0.0, c3 = 0.0;
#pragma unroll
                for (int c = 0; c < C; c += 2) {
                    const uint32_t b0 = (wd[c / 4] >> (8 * (c % 4))) & 0xFFu;
                    const uint32_t b1 = (wd[c / 4] >> (8 * (c % 4) + 8)) & 0xFFu;
                    c0 = fma(qp[c], (double)(b0 >> 4), c0);
                    c1 = fma(qn[c], (double)(b0 & 15u), c1);
                    c2 = fma(qp[c + 1], (double)(b1 >> 4), c2);
                    c3 = fma(qn[c + 1], (double)(b1 & 15u), c3);
                }
                c0 += c2;
                c1 += c3;
            } else {
                const uint32_t wl[4] = {rl[s].x, rl[s].y, rl[s].z, rl[s].w};
                const uint32_t wh[4] = {rh[s].x, rh[s].y, rh[s].z, rh[s].w};
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
            return finish(group_sum_d<LPL>(c0 + c1), rs[s]);
    };
    auto ring = [&](auto slot_score) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) issue(s, s);
        for (int k0 = 0; k0 < K_w; k0 += kRing) {
#pragma unroll
            for (int s = 0; s < kRing; ++s) {
                const int k = k0 + s;
                const double sj = slot_score(s);
                const int j = j0 + lg + k * GROUPS;
                // (no branch: the loads in flight stay countable across iterations)
                s_log[k < K_w && j < j1 && j != j_cur && lane % LPL == 0 ? j - j0 : kMaxRangeLogical + lane] = sj;
                issue(s, k + kRing);              // (past the range: a discarded reload)
            }
        }
    };
    if constexpr (KV_DT == LSA_INT4) {
        if (on_grid) {
            // Exact integer scoring on the matrix cores.  Qp and -Qn are integers
            // below 2^32 on the grid 2^lo; their 7-bit digits (v_mfma_i32_16x16x64_i8
            // takes signed bytes) are the rows of A: rows 0..4 the digits of Qp,
            // rows 8..12 those of -Qn, the other rows zero.  B holds the codes of 16
            // logical pages (its columns): c_max against the A that carries the Qp
            // digits, c_min against the one that carries the -Qn digits, two MFMAs
            // per 64 channels accumulating into one 16 x 16 tile.  Element (r, n) is
            // sum_i digit_r(i) code_i(n) < 2^18; weighted by +-128^d(r) and summed
            // over the rows it is sum_i Qp c_max + Qn c_min of page n in grid steps,
            // an integer below 2^46, so exact in fp64 like every partial sum: the
            // same double as the fp64 path.
            // A lane (row / column lane % 16, k-group kg = lane / 16) supplies the
            // channels 64 hf + 16 kg + e, e = 0..15, of MFMA half hf in A and in B.
            constexpr int NH = D / 64;
            const int rc = lane & 15, kg = lane >> 4;
            int32x4 amax[NH], amin[NH];
            {
                const bool prow = rc < 5, nrow = rc >= 8 && rc < 13;
                const int sh = prow ? 7 * rc : nrow ? 7 * (rc - 8) : 0;
                const uint32_t *src = s_qint + (prow ? 0 : D);
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    uint32_t wp[4] = {0u, 0u, 0u, 0u}, wn[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const uint32_t dg = (src[64 * hf + 16 * kg + e] >> sh) & 127u;
                        wp[e / 4] |= (prow ? dg : 0u) << (8 * (e % 4));
                        wn[e / 4] |= (nrow ? dg : 0u) << (8 * (e % 4));
                    }
                    amax[hf] = int32x4{(int)wp[0], (int)wp[1], (int)wp[2], (int)wp[3]};
                    amin[hf] = int32x4{(int)wn[0], (int)wn[1], (int)wn[2], (int)wn[3]};
                }
            }
            // weight of the tile rows this lane holds (rows 4 kg .. 4 kg + 3)
            double wgt[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 4 * kg + e;
                const int d = rr < 5 ? rr : (rr >= 8 && rr < 13 ? rr - 8 : -1);
                wgt[e] = d < 0 ? 0.0 : ldexp(rr < 8 ? 1.0 : -1.0, 7 * d);
            }
            const double grid = ldexp(1.0, lo);
            // (the fp64 terms die here: keep the first loads below this point)
            __builtin_amdgcn_sched_barrier(0);

            // tiles of 16 logical pages: wavefront w takes tiles w, w + 4, ...,
            // kScoreTiles of them in flight
            constexpr int RT = kScoreTiles;
            const int n_tiles = (j1 - j0 + 15) / 16;
            const int T_w = max(0, (n_tiles - wave + 3) / 4);
            uint4 tb[RT][NH];
            uint32_t tsz[RT];
            auto tissue = [&](int s, int k) __attribute__((always_inline)) {
                int j = j0 + 16 * (wave + 4 * k) + rc;
                if (j >= j1) j = j0;              // past the range: any page of it, discarded
                const unsigned long long hp = s_hp[(j >> gs) - m0];
                const char *st = static_cast<const char *>(a.stats) + (hp << unit_shift) +
                                 ((j & (g - 1)) << row_shift) + 16 * kg;
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) tb[s][hf] = load_stream16(st + 64 * hf);
                tsz[s] = load_stream4(a.k_sz + hp * 2);
                __builtin_amdgcn_sched_barrier(0);   // (in ring order, as above)
            };
#pragma unroll
            for (int s = 0; s < RT; ++s) tissue(s, s);
            for (int k0 = 0; k0 < T_w; k0 += RT) {
#pragma unroll
                for (int s = 0; s < RT; ++s) {
                    const int k = k0 + s;
                    int32x4 acc = {0, 0, 0, 0};
#pragma unroll
                    for (int hf = 0; hf < NH; ++hf) {
                        const uint4 w = tb[s][hf];
                        const int32x4 cmax = {(int)((w.x >> 4) & 0x0F0F0F0Fu), (int)((w.y >> 4) & 0x0F0F0F0Fu),
                                              (int)((w.z >> 4) & 0x0F0F0F0Fu), (int)((w.w >> 4) & 0x0F0F0F0Fu)};
                        const int32x4 cmin = {(int)(w.x & 0x0F0F0F0Fu), (int)(w.y & 0x0F0F0F0Fu),
                                              (int)(w.z & 0x0F0F0F0Fu), (int)(w.w & 0x0F0F0F0Fu)};
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(amax[hf], cmax, acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(amin[hf], cmin, acc, 0, 0, 0);
                    }
                    double part = wgt[0] * (double)acc[0];
#pragma unroll
                    for (int e = 1; e < 4; ++e) part = fma(wgt[e], (double)acc[e], part);
                    const double sj = finish(sum_kgroups_d(part) * grid, tsz[s]);
                    const int j = j0 + 16 * (wave + 4 * k) + rc;
                    s_log[k < T_w && kg == 0 && j < j1 && j != j_cur ? j - j0 : kMaxRangeLogical + lane] = sj;
                    tissue(s, k + RT);            // (past the range: a discarded reload)
                }
            }
        } else {
            ring(fp_slot);                        // terms too wide for one 32-bit grid (rare)
        }
    } else {
        ring(fp_slot);
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

template <int KV_DT, int FPT>
void launch_score_loop_fpt(const ScoreArgs &a, unsigned grid, hipStream_t s) {
    if (a.head_dim == 128) hipLaunchKernelGGL((score_loop_kernel<KV_DT, 128, FPT>), dim3(grid), dim3(kScoreThreads), 0, s, a);
    else hipLaunchKernelGGL((score_loop_kernel<KV_DT, 64, FPT>), dim3(grid), dim3(kScoreThreads), 0, s, a);
}

template <int KV_DT, bool AGG_MAX>
hipError_t launch_score_agg(const ScoreArgs &a, unsigned grid, hipStream_t s) {
    if constexpr (!AGG_MAX) {
        switch (a.fused_pt) {
            case 0: launch_score_loop_fpt<KV_DT, 0>(a, grid, s); break;
            case 4: launch_score_loop_fpt<KV_DT, 4>(a, grid, s); break;
            case 8: launch_score_loop_fpt<KV_DT, 8>(a, grid, s); break;
            case 16: launch_score_loop_fpt<KV_DT, 16>(a, grid, s); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    } else {
        switch (a.fused_pt) {
            case 0: launch_score_fpt<KV_DT, AGG_MAX, 0>(a, grid, s); break;
            case 4: launch_score_fpt<KV_DT, AGG_MAX, 4>(a, grid, s); break;
            case 8: launch_score_fpt<KV_DT, AGG_MAX, 8>(a, grid, s); break;
            case 16: launch_score_fpt<KV_DT, AGG_MAX, 16>(a, grid, s); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
}

template <int KV_DT>
hipError_t launch_score_dt(const ScoreArgs &a, unsigned grid, hipStream_t s) {
    return a.aggregation == LSA_AGG_MAX ? launch_score_agg<KV_DT, true>(a, grid, s)
                                        : launch_score_agg<KV_DT, false>(a, grid, s);
}

}  // namespace

int score_loop_wgs_per_cu(int kv_dtype) { return kv_dtype == LSA_INT4 ? 3 : 2; }

int score_loop_pages_per_block(int batch, int n_ret, int max_pages, int page_size, int logical_page, int kv_dtype) {
    // score_loop_wgs_per_cu workgroups per CU over the chip, within the LDS
    // range limits
    const long long heads = (long long)batch * n_ret;
    const long long slots = (long long)score_loop_wgs_per_cu(kv_dtype) * 256;
    const long long wph = heads >= slots ? 1 : (slots + heads - 1) / heads;
    long long ppb = (max_pages + wph - 1) / wph;
    const int g = page_size / logical_page;
    ppb = ppb < kMaxRangeLogical / g ? ppb : kMaxRangeLogical / g;
    ppb = ppb < kMaxRangePages ? ppb : kMaxRangePages;
    return (int)(ppb < 1 ? 1 : ppb);
}

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

int score_fused_pt(int max_pages, bool agg_max) {
    const int per = (max_pages + kScoreThreads - 1) / kScoreThreads;
    // With the group's scores summed, topk_rows ranks one page past the
    // threads' pages apart, so a sequence of 1025 or 2049 pages (64K tokens
    // plus the decode window at 64-token pages) ranks at 4 or 8 pages per
    // thread instead of 8 or 16: 8 sequences x 4 heads at 64K, 20.5 -> 19.6
    // us per selection call.  At 16 per thread it does not pay: 4097 pages
    // (16 sequences x 4 heads at 256K, int4) ranked in the score kernel that
    // way took 42.4 us per call against 39.8 with the separate kernel (the
    // instance holds 168 VGPRs and spills to scratch in its ranking).
    // (32 pages per thread cost the max-aggregation kernel a wavefront per
    // SIMD; in the sum kernel one 256-thread ranking of 4097 pages at the end
    // took longer than the separate 1024-thread kernel: 62.9 against 51.9 us
    // per int4 selection call at 256K tokens with the radix ranking, 52.7
    // against 39.2 us with the value-binned one, whose 32 scores per thread
    // spill at the 168-register bound)
    const int held = (max_pages - 1 + kScoreThreads - 1) / kScoreThreads;
    if (!agg_max && held <= 8) return held <= 4 ? 4 : 8;
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
    const int per = (a.max_pages - 1 + kTopkThreads - 1) / kTopkThreads;   // (at least 1: max_pages > 4096 here)
    const dim3 g((unsigned)grid), blk(kTopkThreads);
    if (per <= 1) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 1>), g, blk, 0, s, a);
    else if (per <= 2) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 2>), g, blk, 0, s, a);
    else if (per <= 4) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 4>), g, blk, 0, s, a);
    else if (per <= 8) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 8>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((topk_kernel<kTopkThreads, kTopkPerThread>), g, blk, 0, s, a);
    return hipGetLastError();
}

}  // namespace lsa
