// Block-sparse causal prefill attention that visits only non-empty tiles
// (LServe explainer, 技術的詳細 / 統一ブロックスパースアテンション: the kernel
// iterates over the non-empty blocks of a static block pattern, so the cost
// falls with the block sparsity r as 1/(1-r); the figure gives retrieval heads
// a static causal pattern in prefill and streaming heads sink + local blocks;
// 主要な貢献: iterator-based block-sparse kernels).
//
// One workgroup per (KV head, 64-query tile, group of 4 query heads).  The
// workgroup walks the key tiles c that the head's pattern keeps for its query
// tile a (retrieval: c = 0..a; streaming: c < sink_blocks or
// a - c < local_blocks); no dense mask is ever tested.  Each K/V tile is
// staged once in LDS and used by the four query heads of the group (one
// wavefront each), so GQA heads share every K/V read.  The causal mask is
// applied only on the diagonal tile.
//
// Work order.  Workgroups are numbered longest row first (retrieval rows by
// descending a, then the short streaming rows), and consecutive numbers go to
// consecutive XCDs; the head of a workgroup is chosen from its number modulo
// the head count, so the workgroups resident on one XCD share a KV head and
// sweep the same key tiles together, which keeps K/V tiles in that XCD's L2.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 for S^T = K Q^T (keys in M, queries in
// N) and O^T = V^T P^T.  Keys are placed on MFMA rows so that the S^T
// registers of a lane are directly the B operand of the PV product.
#include "lsa_internal.h"

namespace lsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;

struct PItem {
    int kv, a, hg;
    bool streaming;
};

// blockIdx -> (kv head, query tile, head group), longest rows first
__device__ __forceinline__ PItem prefill_item(const PrefillArgs &p) {
    PItem it;
    const int nq = p.n_qblocks, HG = p.head_groups;
    int i = blockIdx.x;
    const int n_ret_items = p.n_ret * nq * HG;
    if (i < n_ret_items) {
        it.kv = p.ret_heads[i % p.n_ret];
        const int j = i / p.n_ret;
        it.hg = j % HG;
        it.a = nq - 1 - j / HG;
        it.streaming = false;
    } else {
        i -= n_ret_items;
        it.kv = p.str_heads[i % p.n_str];
        const int j = i / p.n_str;
        it.hg = j % HG;
        it.a = nq - 1 - j / HG;
        it.streaming = true;
    }
    return it;
}

// visible key tiles of query tile a, ascending: [0, e0) U [s1, a]
__device__ __forceinline__ void tile_ranges(const PrefillArgs &p, const PItem &it, int &e0, int &s1) {
    if (!it.streaming) { e0 = 0; s1 = 0; return; }
    e0 = min(p.sink_blocks, it.a + 1);
    s1 = max(it.a - p.local_blocks + 1, e0);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, head_dim D
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(PrefillArgs p) {
    constexpr int KS = D + 8;          // LDS row stride of K (elements), padded
    constexpr int VS = kTile + 8;      // LDS row stride of V^T (elements), padded
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[kTile * KS];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * VS];

    const PItem it = prefill_item(p);
    int e0, s1;
    tile_ranges(p, it, e0, s1);

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int T = p.seq_len, G = p.group, HQ = p.num_q_heads, NP = p.page_size;
    const int hq_local = it.hg * 4 + wave;          // query head within the group
    const bool head_ok = hq_local < G;
    const int hq = it.kv * G + min(hq_local, G - 1);
    const int col = lane & 31, lg = lane >> 5;      // MFMA column / lane group

    // Q^T as B operand: query 32*qt + col, channels 16*s + 8*lg + j
    bf16x8 qb[2][D / 16];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int row = min(it.a * kTile + 32 * qt + col, T - 1);
        const uint16_t *qrow = static_cast<const uint16_t *>(p.q) + ((size_t)row * HQ + hq) * D;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qb[qt][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qrow + 16 * s + 8 * lg));
    }

    floatx16 o[D / 32][2];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][qt][r] = 0.f;
    float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
    float l_run[2] = {0.f, 0.f};

    // MFMA row rho = 8*ra + 4*rg + rc of a 32-key tile holds key 16*(ra/2) + 8*rg + 4*(ra%2) + rc
    const int rho = lane & 31;
    const int key_of_row = 16 * ((rho >> 3) >> 1) + 8 * ((rho >> 2) & 1) + 4 * ((rho >> 3) & 1) + (rho & 3);

    const uint16_t *kpool = static_cast<const uint16_t *>(p.k);
    const uint16_t *vpool = static_cast<const uint16_t *>(p.v);
    const int n_iter = e0 + (it.a - s1 + 1);
    for (int ii = 0; ii < n_iter; ++ii) {
        const int c = ii < e0 ? ii : s1 + (ii - e0);
        // ---- stage K tile [64][D] and V^T tile [D][64] in LDS (zero keys >= T)
        const int key0 = c * kTile;
        const int pool = p.page_table[key0 / NP];
        const int slot0 = key0 % NP;
        const size_t hp = (size_t)pool * p.num_kv_heads + it.kv;
        __syncthreads();
        {
            constexpr int KCH = kTile * D / 8;      // 16-byte chunks of the K tile
            for (int ch = tid; ch < KCH; ch += 256) {
                const int r = ch / (D / 8), cc = ch % (D / 8);
                uint4 val = make_uint4(0, 0, 0, 0);
                if (key0 + r < T) val = *reinterpret_cast<const uint4 *>(kpool + (hp * NP + slot0 + r) * D + cc * 8);
                *reinterpret_cast<uint4 *>(&k_lds[r * KS + cc * 8]) = val;
            }
            constexpr int VCH = D * kTile / 8;
            for (int ch = tid; ch < VCH; ch += 256) {
                const int d = ch / (kTile / 8), cc = ch % (kTile / 8);
                uint4 val = *reinterpret_cast<const uint4 *>(vpool + (hp * D + d) * NP + slot0 + cc * 8);
                const int kbase = key0 + cc * 8;
                if (kbase + 8 > T) {
                    uint16_t e[8];
                    __builtin_memcpy(e, &val, 16);
#pragma unroll
                    for (int j = 0; j < 8; ++j) if (kbase + j >= T) e[j] = 0;
                    __builtin_memcpy(&val, e, 16);
                }
                *reinterpret_cast<uint4 *>(&v_lds[d * VS + cc * 8]) = val;
            }
        }
        __syncthreads();
        if (!head_ok) continue;

        // ---- S^T = K Q^T : [kt][qt] 32x32 tiles
        floatx16 s[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kt][qt][r] = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const uint16_t *krow = &k_lds[(32 * kt + key_of_row) * KS + 8 * lg];
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(krow + 16 * st));
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[qt][st], s[kt][qt], 0, 0, 0);
            }
        }
        // ---- online softmax per query column; lane holds keys 16*(r/8) + 8*lg + (r%8) of tile kt
        const bool diag = c == it.a;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int qrow = it.a * kTile + 32 * qt + col;
            float mx = -__builtin_inff();
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[kt][qt][r] * p.scale_log2;
                    if (diag) {
                        const int key = key0 + 32 * kt + 16 * (r >> 3) + 8 * lg + (r & 7);
                        if (key > qrow) x = -__builtin_inff();
                    }
                    s[kt][qt][r] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            const float m_new = fmaxf(m_run[qt], mx);
            const float alpha = exp2_fast(m_run[qt] - m_new);
            float ps = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = exp2_fast(s[kt][qt][r] - m_new);
                    s[kt][qt][r] = e;
                    ps += e;
                }
            l_run[qt] = l_run[qt] * alpha + ps;
            m_run[qt] = m_new;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) o[dt][qt] *= alpha;
        }
        // ---- O^T += V^T P^T ; k-step (kt, st): keys 32*kt + 16*st + 8*lg + j
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bf16x8 pb[2];
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    uint32_t pk[4];
#pragma unroll
                    for (int j = 0; j < 8; j += 2)
                        pk[j / 2] = uint32_t(f32_to_bf16_rne(s[kt][qt][8 * st + j])) |
                                    (uint32_t(f32_to_bf16_rne(s[kt][qt][8 * st + j + 1])) << 16);
                    pb[qt] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const bf16x8 va = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4 *>(&v_lds[(32 * dt + col) * VS + 32 * kt + 16 * st + 8 * lg]));
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
                        o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qt], o[dt][qt], 0, 0, 0);
                }
            }
    }

    if (p.tile_counter && tid == 0) {
        const int heads_here = min(4, G - it.hg * 4);
        atomicAdd(p.tile_counter, (unsigned long long)n_iter * heads_here);
    }
    if (!head_ok) return;
    // ---- normalise and store: lane holds query 32*qt + col, channels 32*dt + 8*(r/4) + 4*lg + r%4
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const float lt = l_run[qt] + __shfl_xor(l_run[qt], 32, kWave);
        const float inv = 1.f / lt;
        const int row = it.a * kTile + 32 * qt + col;
        if (row >= T) continue;
        uint16_t *orow = static_cast<uint16_t *>(p.out) + ((size_t)row * HQ + hq) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int d0 = 32 * dt + 8 * rb + 4 * lg;
                uint2 pk;
                pk.x = uint32_t(f32_to_bf16_rne(o[dt][qt][4 * rb] * inv)) |
                       (uint32_t(f32_to_bf16_rne(o[dt][qt][4 * rb + 1] * inv)) << 16);
                pk.y = uint32_t(f32_to_bf16_rne(o[dt][qt][4 * rb + 2] * inv)) |
                       (uint32_t(f32_to_bf16_rne(o[dt][qt][4 * rb + 3] * inv)) << 16);
                *reinterpret_cast<uint2 *>(orow + d0) = pk;
            }
    }
}

// ---------------------------------------------------------------------------
// f32 VALU kernel: lane = query row, wave = query head; K/V tiles in LDS
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs p) {
    extern __shared__ float sm[];
    float *k_lds = sm;                 // [64][D]
    float *v_lds = sm + kTile * D;     // [D][64]

    const PItem it = prefill_item(p);
    int e0, s1;
    tile_ranges(p, it, e0, s1);

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int T = p.seq_len, G = p.group, HQ = p.num_q_heads, NP = p.page_size;
    const int hq_local = it.hg * 4 + wave;
    const bool head_ok = hq_local < G;
    const int hq = it.kv * G + min(hq_local, G - 1);
    const int qrow = it.a * kTile + lane;
    const int qr = min(qrow, T - 1);

    float q[D], o[D];
    const float *qp = static_cast<const float *>(p.q) + ((size_t)qr * HQ + hq) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) { q[d] = qp[d] * p.scale_log2; o[d] = 0.f; }
    float m_run = -__builtin_inff(), l_run = 0.f;

    const float *kpool = static_cast<const float *>(p.k);
    const float *vpool = static_cast<const float *>(p.v);
    const int n_iter = e0 + (it.a - s1 + 1);
    for (int ii = 0; ii < n_iter; ++ii) {
        const int c = ii < e0 ? ii : s1 + (ii - e0);
        const int key0 = c * kTile;
        const int pool = p.page_table[key0 / NP];
        const int slot0 = key0 % NP;
        const size_t hp = (size_t)pool * p.num_kv_heads + it.kv;
        __syncthreads();
        for (int e = tid; e < kTile * D; e += 256) {
            const int r = e / D, d = e % D;
            k_lds[e] = key0 + r < T ? kpool[(hp * NP + slot0 + r) * D + d] : 0.f;
            const int dv = e / kTile, rv = e % kTile;
            v_lds[e] = key0 + rv < T ? vpool[(hp * D + dv) * NP + slot0 + rv] : 0.f;
        }
        __syncthreads();
        if (!head_ok) continue;
        const int nk = min(kTile, qrow - key0 + 1);     // keys p <= t of this tile
        float sc[kTile];
        float mx = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc = fmaf(q[d], k_lds[j * D + d], acc);
            sc[j] = j < nk ? acc : -__builtin_inff();
            mx = fmaxf(mx, sc[j]);
        }
        if (nk <= 0) continue;
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast(m_run - m_new);
        float ps = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float e = j < nk ? exp2_fast(sc[j] - m_new) : 0.f;
            ps += e;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] = fmaf(e, v_lds[d * kTile + j], o[d]);
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;
    }
    if (p.tile_counter && tid == 0) {
        const int heads_here = min(4, G - it.hg * 4);
        atomicAdd(p.tile_counter, (unsigned long long)n_iter * heads_here);
    }
    if (!head_ok || qrow >= T) return;
    float *orow = static_cast<float *>(p.out) + ((size_t)qrow * HQ + hq) * D;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &p, int dtype, hipStream_t s) {
    if (p.n_items == 0) return hipSuccess;
    const dim3 grid((unsigned)p.n_items), block(256);
    if (dtype == LSA_BF16) {
        if (p.head_dim == 128) hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, block, 0, s, p);
        else hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, block, 0, s, p);
    } else {
        // f32 is the small-model path: head_dim 64 only (validated by the caller)
        const size_t lds = 2 * (size_t)kTile * 64 * sizeof(float);
        hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, lds, s, p);
    }
    return hipGetLastError();
}

}  // namespace lsa
