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
#include <type_traits>

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
// bf16 MFMA kernel, head_dim D.  Eight wavefronts: wave w takes query head
// hg*4 + w/2 and query rows 32*(w%2) .. +31 of the tile, so with GQA group 4
// one workgroup covers the tile's four heads and reads each K/V tile once.
// Software pipeline: iteration t issues the QK^T MFMAs of key tile t, then
// runs the softmax and PV of tile t-1, whose VALU work overlaps the QK
// MFMAs in flight.  K tiles and V tiles are double-buffered in LDS separately
// (V lags K by one tile); the global loads of the next tiles are in flight
// during the compute, one barrier per tile.  The last tile is the diagonal
// one: its causal mask is applied in the pipeline's epilogue only.  In LDS,
// key rows are stored in MFMA-row order (the order the QK A operand reads
// them), so the eight lanes of a 128-byte LDS read touch eight consecutive
// padded rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512, 2) void prefill_bf16_kernel(PrefillArgs p) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float floatx2 __attribute__((ext_vector_type(2)));
    constexpr int KS = D + 8;          // LDS row stride of K (elements), padded 16 bytes
    constexpr int VS = kTile + 8;      // LDS row stride of V^T (elements), padded 16 bytes
    constexpr int KCH = kTile * D / 8; // 16-byte chunks of a K tile
    constexpr int VCH = D * kTile / 8; // 16-byte chunks of a V^T tile
    constexpr int NT = 512;
    constexpr int KPT = KCH / NT, VPT = VCH / NT;   // chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kTile * KS];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VS];

    const PItem it = prefill_item(p);
    int e0, s1;
    tile_ranges(p, it, e0, s1);

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int T = p.seq_len, G = p.group, HQ = p.num_q_heads, NP = p.page_size;
    const int hq_local = it.hg * 4 + (wave >> 1);
    const bool head_ok = hq_local < G;
    const int hq = it.kv * G + min(hq_local, G - 1);
    const int q0 = it.a * kTile + 32 * (wave & 1);  // first query row of this wave
    const int col = lane & 31, lg = lane >> 5;      // MFMA column / lane group

    // Q^T as B operand: query q0 + col, channels 16*s + 8*lg + j
    bf16x8 qb[D / 16];
    {
        const int row = min(q0 + col, T - 1);
        const uint16_t *qrow = static_cast<const uint16_t *>(p.q) + ((size_t)row * HQ + hq) * D;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qrow + 16 * s + 8 * lg));
    }

    floatx16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_run = -__builtin_inff();   // running max of the raw scores of query q0 + col
    float l_run = 0.f;                 // this lane's part of the running sum

    const uint16_t *kpool = static_cast<const uint16_t *>(p.k);
    const uint16_t *vpool = static_cast<const uint16_t *>(p.v);
    const int n_iter = e0 + (it.a - s1 + 1);
    auto tile_of = [&](int ii) { return ii < e0 ? ii : s1 + (ii - e0); };
    // A 64-key tile is two whole 32-token blocks of its page, so its keys (and
    // its values) are one contiguous run of 64 * D elements: 16-byte chunk ch of
    // the run is read by consecutive threads, and the chunk's (key, channel
    // group) or (channel, key group) follows from the pool layout.
    auto tile_base = [&](int c) {
        const int key0 = c * kTile;
        const size_t hp = (size_t)p.page_table[key0 / NP] * p.num_kv_heads + it.kv;
        return hp * NP * D + key_offset(key0 % NP, 0, D);       // == value_offset(key0 % NP, 0, D)
    };
    // key chunk ch: tile row r (key), channels 8 * cc .. 8 * cc + 7
    auto k_chunk = [&](int ch, int &r, int &cc) {
        const int rest = ch >> 7;                                // block * (D / 32) + channel slice
        r = 32 * (rest / (D / 32)) + ((ch >> 2) & 31);
        cc = 4 * (rest % (D / 32)) + (ch & 3);
    };
    // value chunk ch: channel d, keys 8 * cc .. 8 * cc + 7 of the tile
    auto v_chunk = [&](int ch, int &d, int &cc) {
        d = (ch >> 2) % D;
        cc = 4 * (ch / (4 * D)) + (ch & 3);
    };

    // Chunk handled by this thread in round e: the wavefront's 64 chunks are
    // one contiguous 1 KiB (16 rows x 4 chunks).  Lane l takes chunk column
    // l / 16 of row l % 16 (values) or of the key row that lands on LDS row
    // l % 16 (keys: the MFMA-order row permutation swaps bits 2 and 3 of the
    // key), so consecutive lanes store to consecutive padded LDS rows and a
    // write phase touches distinct banks.
    const int r16 = lane & 15;
    const int k_lane_chunk = 4 * ((r16 & 3) | ((r16 & 4) << 1) | ((r16 & 8) >> 1)) + (lane >> 4);
    const int v_lane_chunk = 4 * r16 + (lane >> 4);
    auto chunk_k = [&](int e) { return (wave + e * (NT / kWave)) * kWave + k_lane_chunk; };
    auto chunk_v = [&](int e) { return (wave + e * (NT / kWave)) * kWave + v_lane_chunk; };

    // global -> registers (keys >= T read as zero); registers -> LDS
    uint4 kreg[KPT], vreg[VPT];
    auto fetch_k = [&](int ii) {
        const int c = tile_of(ii);
        const uint16_t *src = kpool + tile_base(c);
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int ch = chunk_k(e);
            int r, cc;
            k_chunk(ch, r, cc);
            kreg[e] = c * kTile + r < T ? *reinterpret_cast<const uint4 *>(src + (size_t)ch * 8) : make_uint4(0, 0, 0, 0);
        }
    };
    auto fetch_v = [&](int ii) {
        const int c = tile_of(ii);
        const uint16_t *src = vpool + tile_base(c);
#pragma unroll
        for (int e = 0; e < VPT; ++e) {
            const int ch = chunk_v(e);
            int d, cc;
            v_chunk(ch, d, cc);
            uint4 val = *reinterpret_cast<const uint4 *>(src + (size_t)ch * 8);
            const int kbase = c * kTile + cc * 8;
            if (kbase + 8 > T) {
                const int nv = T - kbase;          // valid keys in this chunk (<= 7)
                uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2)
                    w[q2] &= (2 * q2 < nv ? 0x0000FFFFu : 0u) | (2 * q2 + 1 < nv ? 0xFFFF0000u : 0u);
                val = make_uint4(w[0], w[1], w[2], w[3]);
            }
            vreg[e] = val;
        }
    };
    auto stash_k = [&](int buf) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int ch = chunk_k(e);
            int key, cc;
            k_chunk(ch, key, cc);
            // key k of a 32-key half is stored at the LDS row of the MFMA row that reads it
            const int kk = key & 31;
            const int rho = 8 * (2 * (kk >> 4) + ((kk >> 2) & 1)) + 4 * ((kk >> 3) & 1) + (kk & 3);
            *reinterpret_cast<uint4 *>(&k_lds[buf][((key & 32) + rho) * KS + cc * 8]) = kreg[e];
        }
    };
    auto stash_v = [&](int buf) {
#pragma unroll
        for (int e = 0; e < VPT; ++e) {
            const int ch = chunk_v(e);
            int d, cc;
            v_chunk(ch, d, cc);
            *reinterpret_cast<uint4 *>(&v_lds[buf][d * VS + cc * 8]) = vreg[e];
        }
    };

    const float sc = p.scale_log2;
    // S^T = K Q^T of the tile in K buffer kb: lane holds keys 32*kt + 16*(r/8) + 8*lg + r%8, query q0 + col
    auto qk = [&](int kb, floatx16 (&s)[2]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const uint16_t *krow = &k_lds[kb][(32 * kt + col) * KS + 8 * lg];
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(krow)), qb[0], floatx16{}, 0, 0, 0);
#pragma unroll
            for (int st = 1; st < D / 16; ++st) {
                const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(krow + 16 * st));
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[st], s[kt], 0, 0, 0);
            }
        }
    };
    // online softmax of the scores s (DIAG: causal mask against key0), then O^T += V^T P^T
    auto softmax_pv = [&](floatx16 (&s)[2], int vb, int key0, auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        if constexpr (DIAG) {
            const int qrow = q0 + col;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (key0 + 32 * kt + 16 * (r >> 3) + 8 * lg + (r & 7) > qrow) s[kt][r] = -__builtin_inff();
        }
        float mx = s[0][0];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        mx = max_xor32(mx);
        const float m_new = fmaxf(m_run, mx);
        if (__ballot(m_new > m_run) != 0) {            // rescale only when some column's max moved
            const float alpha = exp2_fast((m_run - m_new) * sc);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
            m_run = m_new;
        }
        const float mb = m_run * sc;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                uint32_t pk[4];
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const float e0v = exp2_fast(fmaf(s[kt][8 * st + j], sc, -mb));
                    const float e1v = exp2_fast(fmaf(s[kt][8 * st + j + 1], sc, -mb));
                    l_run += e0v + e1v;
                    pk[j / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{e0v, e1v}, bf16x2));
                }
                const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
                // k-step (kt, st): keys 32*kt + 16*st + 8*lg + j
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const bf16x8 va = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4 *>(&v_lds[vb][(32 * dt + col) * VS + 32 * kt + 16 * st + 8 * lg]));
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dt], 0, 0, 0);
                }
            }
    };

    // prologue: K(0) in LDS
    fetch_k(0);
    stash_k(0);
    __syncthreads();
    floatx16 sa[2], sb[2];                           // scores of even / odd tiles
    auto step = [&](int ii, floatx16 (&s_cur)[2], floatx16 (&s_prev)[2]) {
        // in flight during the compute: K(ii+1) and V(ii)
        if (ii + 1 < n_iter) fetch_k(ii + 1);
        fetch_v(ii);
        if (head_ok) {
            qk(ii & 1, s_cur);
            if (ii > 0) softmax_pv(s_prev, (ii - 1) & 1, tile_of(ii - 1) * kTile, std::false_type{});
        }
        if (ii + 1 < n_iter) stash_k((ii + 1) & 1);
        stash_v(ii & 1);
        __syncthreads();
    };
    int ii = 0;
    for (; ii + 1 < n_iter; ii += 2) {
        step(ii, sa, sb);
        step(ii + 1, sb, sa);
    }
    if (ii < n_iter) step(ii, sa, sb);
    // epilogue: the last tile (the diagonal one)
    if (head_ok) {
        if ((n_iter - 1) & 1) softmax_pv(sb, (n_iter - 1) & 1, tile_of(n_iter - 1) * kTile, std::true_type{});
        else softmax_pv(sa, (n_iter - 1) & 1, tile_of(n_iter - 1) * kTile, std::true_type{});
    }

    if (p.tile_counter && tid == 0) {
        const int heads_here = min(4, G - it.hg * 4);
        atomicAdd(p.tile_counter, (unsigned long long)n_iter * heads_here);
    }
    if (!head_ok) return;
    // ---- normalise and store: lane holds query q0 + col, channels 32*dt + 8*(r/4) + 4*lg + r%4
    const float lt = sum_xor32(l_run);
    const float inv = 1.f / lt;
    const int row = q0 + col;
    if (row >= T) return;
    uint16_t *orow = static_cast<uint16_t *>(p.out) + ((size_t)row * HQ + hq) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int d0 = 32 * dt + 8 * rb + 4 * lg;
            const bf16x2 a01 = __builtin_convertvector(floatx2{o[dt][4 * rb] * inv, o[dt][4 * rb + 1] * inv}, bf16x2);
            const bf16x2 a23 = __builtin_convertvector(floatx2{o[dt][4 * rb + 2] * inv, o[dt][4 * rb + 3] * inv}, bf16x2);
            uint2 pk;
            pk.x = __builtin_bit_cast(uint32_t, a01);
            pk.y = __builtin_bit_cast(uint32_t, a23);
            *reinterpret_cast<uint2 *>(orow + d0) = pk;
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
            k_lds[e] = key0 + r < T ? kpool[hp * NP * D + key_offset(slot0 + r, d, D)] : 0.f;
            const int dv = e / kTile, rv = e % kTile;
            v_lds[e] = key0 + rv < T ? vpool[hp * NP * D + value_offset(slot0 + rv, dv, D)] : 0.f;
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
        if (p.head_dim == 128) hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(512), 0, s, p);
        else hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, dim3(512), 0, s, p);
    } else {
        // f32 is the small-model path: head_dim 64 only (validated by the caller)
        const size_t lds = 2 * (size_t)kTile * 64 * sizeof(float);
        hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, lds, s, p);
    }
    return hipGetLastError();
}

}  // namespace lsa
