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
//
// Top-K.  Scores are mapped to order-preserving 64-bit keys; a most
// significant digit first radix select (8-bit digits, histogram in LDS) finds
// the K-th largest key; equal keys are taken in ascending page order (ties
// to the lower page index); an ordered compaction writes the selected pages
// in ascending order.
#include "lsa_internal.h"

namespace lsa {
namespace {

template <int EB, int D>
struct ScoreShape {
    static constexpr int C = 16 / EB;        // channels per lane (one 16-byte load)
    static constexpr int LPL = D / C;        // lanes per logical page
    static constexpr int LPP = kWave / LPL;  // logical pages per pass
};

__device__ __forceinline__ double shfl_xor_d(double v, int m) { return __shfl_xor(v, m, kWave); }

// Qp / Qn of this lane's channels, fp64.
template <int C>
__device__ __forceinline__ void load_q_pos_neg(const ScoreArgs &a, int b, int kv, int ch0,
                                                double (&qp)[C], double (&qn)[C]) {
    const int G = a.num_q_heads / a.num_kv_heads;
#pragma unroll
    for (int c = 0; c < C; ++c) { qp[c] = 0.0; qn[c] = 0.0; }
    for (int h = 0; h < G; ++h) {
        const size_t row = ((size_t)b * a.num_q_heads + (size_t)kv * G + h) * a.head_dim + ch0;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            double x;
            if (a.q_dtype == LSA_BF16) x = (double)bf16_to_f32(static_cast<const uint16_t *>(a.q)[row + c]);
            else x = (double)static_cast<const float *>(a.q)[row + c];
            qp[c] += fmax(x, 0.0);
            qn[c] += fmin(x, 0.0);
        }
    }
}

// KV_DT: LSA_F32, LSA_BF16 (stats in that type) or LSA_INT4 (code stats).
template <int KV_DT, int D>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    constexpr int EB = KV_DT == LSA_F32 ? 4 : (KV_DT == LSA_BF16 ? 2 : 1);
    using S = ScoreShape<EB, D>;
    constexpr int C = S::C, LPL = S::LPL, LPP = S::LPP;

    const int blk = blockIdx.x % a.blocks_per_head;
    const int rest = blockIdx.x / a.blocks_per_head;
    const int r = rest % a.n_ret;
    const int b = rest / a.n_ret;
    const int kv = a.ret_heads[r];
    const int L = a.seq_lens[b];
    const int n_pages = (L + a.page_size - 1) / a.page_size;
    const int m0 = blk * a.pages_per_block;
    if (m0 >= n_pages) return;
    const int m1 = min(m0 + a.pages_per_block, n_pages);

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int lg = lane / LPL;              // lane group = logical page within a pass
    const int ch0 = (lane % LPL) * C;

    double qp[C], qn[C];
    load_q_pos_neg<C>(a, b, kv, ch0, qp, qn);
    double qsum = 0.0;                      // int4 only: sum over all channels of Qp + Qn
    if constexpr (KV_DT == LSA_INT4) {
#pragma unroll
        for (int c = 0; c < C; ++c) qsum += qp[c] + qn[c];
#pragma unroll
        for (int off = 1; off < LPL; off <<= 1) qsum += shfl_xor_d(qsum, off);
    }

    const int g = a.page_size / a.logical_page;
    const int ge = min(g, LPP);             // lane groups per physical page in one pass
    const int ppp = LPP / ge;               // physical pages per pass
    const int npass = g / ge;               // passes per physical page
    const size_t head_stride = (size_t)g * (KV_DT == LSA_INT4 ? D : 2 * D);

    for (int mp = m0 + wave * ppp; mp < m1; mp += 4 * ppp) {
        const int m = mp + lg / ge;
        const bool page_ok = m < m1;
        int pool = 0;
        double s_scale = 1.0, s_zero = 0.0;
        if (page_ok) {
            pool = a.page_table[(size_t)b * a.max_pages + m];
            if constexpr (KV_DT == LSA_INT4) {
                const uint16_t *sz = a.k_sz + ((size_t)pool * a.num_kv_heads + kv) * 2;
                s_scale = (double)fp16_bits_to_f32(sz[0]);
                s_zero = (double)fp16_bits_to_f32(sz[1]);
            }
        }
        double best = -__builtin_inf();
        for (int pass = 0; pass < npass; ++pass) {
            const int jl = pass * ge + lg % ge;             // logical page within physical page
            const int j = m * g + jl;
            const bool ok = page_ok && j * a.logical_page < L;
            double acc = 0.0;
            if (ok) {
                const size_t base = ((size_t)pool * a.num_kv_heads + kv) * head_stride;
                if constexpr (KV_DT == LSA_INT4) {
                    const uint8_t *st = static_cast<const uint8_t *>(a.stats) + base + (size_t)jl * D + ch0;
                    const uint4 w = *reinterpret_cast<const uint4 *>(st);
                    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const uint32_t byte = (wd[c / 4] >> (8 * (c % 4))) & 0xFFu;
                        acc = fma(qp[c], (double)(byte >> 4), acc);
                        acc = fma(qn[c], (double)(byte & 15u), acc);
                    }
                } else if constexpr (KV_DT == LSA_BF16) {
                    const uint16_t *st = static_cast<const uint16_t *>(a.stats) + base + (size_t)jl * 2 * D + ch0;
                    const uint4 lo = *reinterpret_cast<const uint4 *>(st);
                    const uint4 hi = *reinterpret_cast<const uint4 *>(st + D);
                    const uint32_t wl[4] = {lo.x, lo.y, lo.z, lo.w};
                    const uint32_t wh[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const float kmin = (c & 1) ? bf16_hi(wl[c / 2]) : bf16_lo(wl[c / 2]);
                        const float kmax = (c & 1) ? bf16_hi(wh[c / 2]) : bf16_lo(wh[c / 2]);
                        acc = fma(qp[c], (double)kmax, acc);
                        acc = fma(qn[c], (double)kmin, acc);
                    }
                } else {
                    const float *st = static_cast<const float *>(a.stats) + base + (size_t)jl * 2 * D + ch0;
                    const float4 lo = *reinterpret_cast<const float4 *>(st);
                    const float4 hi = *reinterpret_cast<const float4 *>(st + D);
                    const float vl[4] = {lo.x, lo.y, lo.z, lo.w};
                    const float vh[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        acc = fma(qp[c], (double)vh[c], acc);
                        acc = fma(qn[c], (double)vl[c], acc);
                    }
                }
            }
#pragma unroll
            for (int off = 1; off < LPL; off <<= 1) acc += shfl_xor_d(acc, off);
            double sj = acc;
            if constexpr (KV_DT == LSA_INT4) sj = s_scale * (acc - s_zero * qsum);
            if (!ok) sj = -__builtin_inf();
            // max over the lane groups that hold logical pages of the same physical page
            for (int off = LPL; off < ge * LPL; off <<= 1) sj = fmax(sj, shfl_xor_d(sj, off));
            best = fmax(best, sj);
        }
        if (page_ok && (lane % (ge * LPL)) == 0)
            a.phys[((size_t)b * a.num_kv_heads + kv) * a.max_pages + m] = best + 0.0;
    }
}

// ---------------------------------------------------------------------------
// top-K: one workgroup of 256 threads per (sequence, retrieval head)
// ---------------------------------------------------------------------------

__device__ __forceinline__ unsigned long long order_key(double x) {
    x = x + 0.0;                                  // -0 -> +0
    const unsigned long long u = __double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// inclusive prefix sum over the 256 threads of a 32-bit packed counter
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t *wave_tot) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t n = __shfl_up(v, off, kWave);
        if (lane >= off) v += n;
    }
    if (lane == kWave - 1) wave_tot[wave] = v;
    __syncthreads();
    uint32_t add = 0;
    for (int w = 0; w < wave; ++w) add += wave_tot[w];
    __syncthreads();
    return v + add;
}

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_digit, sh_above;
    __shared__ uint32_t wave_tot[4];

    const int r = blockIdx.x % a.n_ret;
    const int b = blockIdx.x / a.n_ret;
    const int kv = a.ret_heads[r];
    const int L = a.seq_lens[b];
    const int n = (L + a.page_size - 1) / a.page_size;
    const int K = a.k;
    int32_t *out = a.selected + ((size_t)b * a.num_kv_heads + kv) * K;
    const double *P = a.phys + ((size_t)b * a.num_kv_heads + kv) * a.max_pages;
    const int tid = threadIdx.x;

    if (n <= K) {                                 // every page, ascending, padded with -1
        for (int i = tid; i < K; i += blockDim.x) out[i] = i < n ? i : -1;
        return;
    }

    unsigned long long prefix = 0, mask = 0;
    uint32_t need = (uint32_t)K;
    for (int shift = 56; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += blockDim.x) {
            const unsigned long long key = order_key(P[i]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFFu], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l owns bins 4l..4l+3; suffix sums from the top bin down
            const uint32_t c0 = hist[4 * tid], c1 = hist[4 * tid + 1], c2 = hist[4 * tid + 2], c3 = hist[4 * tid + 3];
            const uint32_t mine = c0 + c1 + c2 + c3;
            uint32_t suf = mine;                  // inclusive suffix sum over lanes >= tid
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t nb = __shfl_down(suf, off, kWave);
                if (tid + off < kWave) suf += nb;
            }
            uint32_t above = suf - mine;          // elements in bins of higher lanes
            const uint32_t cs[4] = {c0, c1, c2, c3};
            for (int q = 3; q >= 0; --q) {
                if (above < need && above + cs[q] >= need) {
                    sh_digit = 4 * tid + q;
                    sh_above = above;
                }
                above += cs[q];
            }
        }
        __syncthreads();
        const uint32_t d = sh_digit;
        need -= sh_above;
        prefix |= (unsigned long long)d << shift;
        mask |= 0xFFull << shift;
        const bool done = hist[d] == need;        // the whole bin is taken
        __syncthreads();
        if (done) break;
    }

    // ordered compaction: thread t owns the contiguous segment [t*seg, (t+1)*seg)
    const int seg = (n + blockDim.x - 1) / blockDim.x;
    const int i0 = min(n, tid * seg), i1 = min(n, i0 + seg);
    uint32_t cnt = 0;                             // low 16 bits: greater, high 16 bits: equal
    for (int i = i0; i < i1; ++i) {
        const unsigned long long km = order_key(P[i]) & mask;
        cnt += km > prefix ? 1u : (km == prefix ? 0x10000u : 0u);
    }
    const uint32_t incl = block_inclusive_scan(cnt, wave_tot);
    uint32_t gt_before = (incl - cnt) & 0xFFFFu;
    uint32_t eq_before = (incl - cnt) >> 16;
    for (int i = i0; i < i1; ++i) {
        const unsigned long long km = order_key(P[i]) & mask;
        if (km > prefix) {
            out[gt_before + min(eq_before, need)] = i;
            ++gt_before;
        } else if (km == prefix) {
            if (eq_before < need) out[gt_before + eq_before] = i;
            ++eq_before;
        }
    }
}

template <int KV_DT>
hipError_t launch_score_dt(const ScoreArgs &a, unsigned grid, hipStream_t s) {
    if (a.head_dim == 128) hipLaunchKernelGGL((score_kernel<KV_DT, 128>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((score_kernel<KV_DT, 64>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

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
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace lsa
