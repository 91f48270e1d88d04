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
// wavefront pair each), so GQA heads share every K/V read.  The causal mask is
// applied only on the diagonal tile.  With fewer than four query heads per KV
// head (G = 1 or 2) a workgroup takes 4 / G consecutive query tiles of its KV
// head instead, walks the union of their key tiles, and each wavefront pair
// computes only the tiles its own query tile sees, so no wavefront idles.
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

#include <type_traits>

namespace lsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;

// 16 bytes per lane from base + voff into LDS (the wavefront's 64 lanes fill
// 1 KiB at lds), through a raw buffer resource of `bytes` bytes at base: a
// lane whose offset falls outside it reads zeros instead of memory.
__device__ __forceinline__ void buffer_to_lds16(const void *base, int bytes, uint32_t voff, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(base, bytes), (void __attribute__((address_space(3))) *)lds,
                                             16, voff, 0, 0, 0);
}

struct PItem {
    int kv, a, hg;
    bool streaming;
};

// blockIdx -> (kv head, query tile, head group), longest rows first.
// Workgroups are handed to the XCDs in number order, round robin, so each
// round of consecutive numbers should hold rows of equal length: a round that
// mixes long and short rows leaves the XCDs of the short ones waiting for the
// others.  Head-kind patterns order rows by a and kind.  A static block mask
// comes with its own order (rows sorted by length, computed once per mask);
// without one, the head of consecutive workgroups rotates every round.
template <bool CSR, int QT>
__device__ __forceinline__ PItem prefill_item(const PrefillArgs &p) {
    PItem it;
    const int nq = p.n_qblocks, HG = p.head_groups, NG = p.n_qgroups;
    int i = blockIdx.x;
    if (CSR && p.order) {
        // one code per (KV head, query tile, head group); with QT > 1 a code
        // stands for the group of QT query tiles that holds its tile, and the
        // grid reads only the leading entries, which the schedule fills with
        // one code per group
        const int code = min(max(p.order[i], 0), p.n_ret * nq * HG - 1);
        it.hg = code % HG;
        it.a = (code / HG) % nq;
        it.kv = code / (HG * nq);
        it.streaming = false;
        if (QT > 1) it.a = nq - 1 - ((nq - 1 - it.a) / QT) * QT;
        return it;
    }
    // it.a is the highest query tile of the item (its QT tiles are it.a - QT + 1 .. it.a)
    const int n_ret_items = p.n_ret * NG * HG;
    if (i < n_ret_items) {
        if (!CSR && p.n_ret > kXcds && p.n_ret % kXcds == 0) {
            // more retrieval heads than XCDs: XCD x (workgroup i % 8) takes
            // heads x, x + 8, ... one after the other, each longest rows
            // first, so the workgroups that share an L2 stream one head's
            // tiles together (multi-head layer, 16 retrieval heads: 73.1-73.4
            // -> 70.8-72.0 ms against two heads interleaved per XCD)
            const int x = i % kXcds, r = i / kXcds, per = NG * HG;
            const int j = r % per;
            it.kv = p.ret_heads[x + kXcds * (r / per)];
            it.hg = j % HG;
            it.a = nq - 1 - (j / HG) * QT;
        } else {
            const int j = i / p.n_ret;
            it.kv = p.ret_heads[CSR ? (i + j) % p.n_ret : i % p.n_ret];
            it.hg = j % HG;
            it.a = nq - 1 - (j / HG) * QT;
        }
        it.streaming = false;
    } else {
        i -= n_ret_items;
        it.kv = p.str_heads[i % p.n_str];
        const int j = i / p.n_str;
        it.hg = j % HG;
        it.a = nq - 1 - (j / HG) * QT;
        it.streaming = true;
    }
    return it;
}

// The key tiles a work item visits, ascending.  Head-kind patterns: [0, e0)
// U [s1, a].  Static block masks: entries rp0 .. rp0 + n - 1 of col_idx; the
// row offsets are clamped to [0, nnz] and the tiles to [0, a], so a malformed
// mask cannot make the kernel read outside the arrays or the sequence.
struct TileRow {
    int e0, s1, rp0, n;
};

template <bool CSR, int QT>
__device__ __forceinline__ TileRow tile_row(const PrefillArgs &p, const PItem &it) {
    TileRow r{0, 0, 0, 0};
    if constexpr (CSR && QT > 1) {
        return r;                                 // the union of the item's rows is built in LDS
    } else if constexpr (CSR) {
        const int32_t *rp = p.row_ptr + (size_t)it.kv * (p.n_qblocks + 1) + it.a;
        const int b0 = min(max(rp[0], 0), p.nnz);
        const int b1 = min(max(rp[1], b0), p.nnz);
        r.rp0 = b0;
        r.n = b1 - b0;
    } else {
        if (it.streaming) {                       // the union over the item's query tiles
            r.e0 = min(p.sink_blocks, it.a + 1);
            r.s1 = max(max(it.a - QT + 1, 0) - p.local_blocks + 1, r.e0);
        }
        r.n = r.e0 + (it.a - r.s1 + 1);
    }
    return r;
}

template <bool CSR>
__device__ __forceinline__ int row_tile(const PrefillArgs &p, const PItem &it, const TileRow &r, int ii) {
    if constexpr (CSR) return min(max(p.col_idx[r.rp0 + ii], 0), it.a);
    else return ii < r.e0 ? ii : r.s1 + (ii - r.e0);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, head_dim D.  Eight wavefronts: wave w takes query head
// hg*4 + w/2 and query rows 32*(w%2) .. +31 of the tile, so with GQA group 4
// one workgroup covers the tile's four heads and reads each K/V tile once.
// Step t runs the softmax of key tile t-1 (VALU phase), then its PV product
// and the QK^T MFMAs of tile t (MFMA phase); waves 4-7 run one phase behind
// waves 0-3, so the two wavefronts of each SIMD alternate between the
// phases.  K and V tiles sit in a four-deep LDS ring, loaded from global
// memory straight into LDS (global_load_lds_dwordx4: no registers, no LDS
// store instructions) two tiles (K) and one tile (V) ahead of their use.
// The last tile is the diagonal one: its causal mask is applied in the
// epilogue only.
// ---------------------------------------------------------------------------
template <int D, bool CSR, int QT>
__global__ __launch_bounds__(512, 2) void prefill_bf16_kernel(PrefillArgs p) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float floatx2 __attribute__((ext_vector_type(2)));
    constexpr int NT = 512;
    constexpr int NS = D / 32;                        // 32-channel slices of a key row
    constexpr int KPT = kTile * D / 8 / NT;           // 16-byte chunks per thread and tile
    // LDS tiles mirror the pool's blocks: K as [2 blocks][D/32 slices][32 rows][32 channels],
    // V as [2 blocks][D channels][32 tokens]; 16-byte chunk c of a 64-byte row r sits at
    // position c ^ ((r >> 2) & 3) of its row (row = key for K, channel for V), which keeps
    // the MFMA operand reads free of bank conflicts.
    // A ring of four K and four V tiles: step ii computes on K(ii) and V(ii-1)
    // while K(ii+2) and V(ii+1) land, so a fetch has two steps to arrive.  Each
    // buffer is an LDS object of its own and the steps are unrolled by four, so
    // the compiler can tell that the tile being read is not one that a fetch
    // in flight writes (else it waits for every fetch before each read).
    __shared__ __attribute__((aligned(16))) uint16_t k_lds0[kTile * D], k_lds1[kTile * D], k_lds2[kTile * D],
        k_lds3[kTile * D];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds0[kTile * D], v_lds1[kTile * D], v_lds2[kTile * D],
        v_lds3[kTile * D];
    auto kbuf = [&](auto b) -> uint16_t * {
        constexpr int i = decltype(b)::value & 3;
        if constexpr (i == 0) return k_lds0;
        else if constexpr (i == 1) return k_lds1;
        else if constexpr (i == 2) return k_lds2;
        else return k_lds3;
    };
    auto vbuf = [&](auto b) -> uint16_t * {
        constexpr int i = decltype(b)::value & 3;
        if constexpr (i == 0) return v_lds0;
        else if constexpr (i == 1) return v_lds1;
        else if constexpr (i == 2) return v_lds2;
        else return v_lds3;
    };

    const PItem it = prefill_item<CSR, QT>(p);
    const TileRow trow = tile_row<CSR, QT>(p, it);

    const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int T = p.seq_len, G = p.group, HQ = p.num_q_heads, NP = p.page_size;
    // wavefront pair `slot`: query head and query tile; with QT > 1 the group is G = 4 / QT
    const int slot = wave >> 1;
    constexpr int GQ = QT > 1 ? 4 / QT : 1;
    const int hq_local = QT == 1 ? it.hg * 4 + slot : slot % GQ;
    const int a_s = QT == 1 ? it.a : it.a - slot / GQ;        // this pair's query tile
    const bool head_ok = QT == 1 ? hq_local < G : a_s >= 0;
    const int hq = it.kv * G + min(hq_local, G - 1);
    const int q0 = max(a_s, 0) * kTile + 32 * (wave & 1);   // first query row of this wave
    // A static mask with QT > 1: the item walks the union of its query tiles'
    // rows.  Each row marks its tiles in a bitmap of its own; the union is
    // then compacted in ascending order into u_list, each entry the tile in
    // bits 0..23 and, in bits 24..27, which of the QT query tiles list it.
    // Elsewhere an entry is just the tile.
    constexpr bool kUnion = CSR && QT > 1;
    int n_union = 0;
    int *u_list = nullptr;
    if constexpr (kUnion) {
        __shared__ int u_entries[kPrefillMaxUnionTiles];
        __shared__ uint32_t u_bits[QT][kPrefillMaxUnionTiles / 32];
        __shared__ uint32_t u_wtot[NT / kWave];
        u_list = u_entries;
        const int words = (it.a + 32) / 32;                  // tiles 0 .. it.a
        for (int e = tid; e < QT * words; e += NT) u_bits[e / words][e % words] = 0;
        __syncthreads();
#pragma unroll
        for (int si = 0; si < QT; ++si) {
            const int ar = it.a - si;
            if (ar < 0) break;
            const int32_t *rp = p.row_ptr + (size_t)it.kv * (p.n_qblocks + 1) + ar;
            const int b0 = min(max(rp[0], 0), p.nnz);
            const int b1 = min(max(rp[1], b0), p.nnz);
            for (int e = b0 + tid; e < b1; e += NT) {
                const int c = min(max(p.col_idx[e], 0), ar);
                atomicOr(&u_bits[si][c >> 5], 1u << (c & 31));
            }
        }
        __syncthreads();
        uint32_t uw = 0, cnt = 0;
        if (tid < words) {
#pragma unroll
            for (int si = 0; si < QT; ++si) uw |= u_bits[si][tid];
            cnt = __popc(uw);
        }
        const uint32_t incl = wave_inclusive_scan(cnt);
        if (lane == kWave - 1) u_wtot[wave] = incl;
        __syncthreads();
        uint32_t off = incl - cnt, total = 0;
#pragma unroll
        for (int w2 = 0; w2 < NT / kWave; ++w2) {
            off += w2 < wave ? u_wtot[w2] : 0;
            total += u_wtot[w2];
        }
        while (uw) {
            const int bit = __builtin_ctz(uw);
            uw &= uw - 1;
            uint32_t mem = 0;
#pragma unroll
            for (int si = 0; si < QT; ++si) mem |= ((u_bits[si][tid] >> bit) & 1u) << si;
            u_list[off++] = (32 * tid + bit) | (int)(mem << 24);
        }
        n_union = (int)total;
        __syncthreads();
    }
    auto tile_id = [&](int v) { return kUnion ? (v & 0xFFFFFF) : v; };
    // does this pair's query tile see key tile entry v (QT > 1: the item walks a union)
    auto sees = [&](int v) {
        if constexpr (kUnion) return ((v >> (24 + slot / GQ)) & 1) != 0;
        return v <= a_s && (!it.streaming || v < p.sink_blocks || a_s - v < p.local_blocks);
    };
    const int col = lane & 31, lg = lane >> 5;      // MFMA column / lane group
    const int n_iter = kUnion ? n_union : trow.n;
    if (n_iter == 0) {                              // a query tile without key tiles: zero output
        const int row = q0 + col;
        if (!head_ok || row >= T) return;
        uint16_t *orow = static_cast<uint16_t *>(p.out) + ((size_t)row * HQ + hq) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) *reinterpret_cast<uint2 *>(orow + 32 * dt + 8 * rb + 4 * lg) = make_uint2(0, 0);
        return;
    }

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
    // Static masks: the row's column indices are read with scalar loads
    // (constant address space, like the page table below), which the tile
    // fetches in flight do not delay; ii < n_iter always.
    const int32_t __attribute__((address_space(4))) *cidx =
        (const int32_t __attribute__((address_space(4))) *)p.col_idx + trow.rp0;
    auto tile_of = [&](int ii) {
        if constexpr (kUnion) {
            return __builtin_amdgcn_readfirstlane(u_list[ii]);
        } else if constexpr (CSR) {
            return min(max((int)cidx[ii], 0), it.a);
        } else {
            return row_tile<false>(p, it, trow, ii);
        }
    };
    // A 64-key tile is two whole 32-token blocks of its page: its keys (and its
    // values) are one contiguous run of 64 * D elements laid out like the LDS tile.
    // The page table is read through the constant address space: a scalar
    // load, counted apart from the vector loads, so the lookup does not wait
    // for the tile fetches in flight (a vector load here made every step wait
    // for the K tile it had just requested).  Nothing writes the table while
    // the kernel runs.
    const int32_t __attribute__((address_space(4))) *ptab =
        (const int32_t __attribute__((address_space(4))) *)p.page_table;
    auto tile_base = [&](int c) {
        const int key0 = c * kTile;
        const size_t hp = (size_t)ptab[key0 / NP] * p.num_kv_heads + it.kv;
        return hp * NP * D + key_offset(key0 % NP, 0, D);       // == value_offset(key0 % NP, 0, D)
    };
    auto swz = [](int r) { return (r >> 2) & 3; };

    // global -> LDS without registers: wavefront instruction j fills LDS chunks
    // 64j .. 64j+63 (16 rows of 4 chunks); lane l writes position l, i.e. row
    // 16j + l/4, position l%4, and so reads the row's logical chunk
    // (l%4) ^ swz(row) from the pool: one contiguous 1 KiB per instruction.
    // The fetch is a raw buffer load into LDS: the tile's base goes in a
    // buffer resource (scalar registers) whose size is the tile's, so no access
    // leaves the tile, and the lane's byte offset within the tile, the same
    // for every tile, is formed once.
    uint32_t fetch_off[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const int j = wave + e * (NT / kWave);
        const int row = 16 * j + (lane >> 2);                    // (block, slice, key) or (block, channel) row
        const int c = (lane & 3) ^ swz(row);                     // swz(row) = swz(row % 32) = swz(channel)
        fetch_off[e] = (uint32_t)(row * 32 + c * 8) * 2u;
    }
    auto fetch = [&](const uint16_t *pool, uint16_t *lds, size_t base) {
#pragma unroll
        for (int e = 0; e < KPT; ++e)
            buffer_to_lds16(pool + base, kTile * D * (int)sizeof(uint16_t), fetch_off[e],
                            lds + (wave + e * (NT / kWave)) * 512);
    };
    // values of keys >= T (only in the sequence's last tile) may hold any bits:
    // zero them once they have landed, so a zero probability never meets a NaN
    auto zero_v_tail = [&](uint16_t *vl, int key0) {
        if (key0 + kTile <= T) return;
        for (int e = tid; e < 2 * D * 32; e += NT) {
            const int blk = e / (D * 32), ch = (e / 32) % D, t = e % 32;
            if (key0 + 32 * blk + t >= T)
                vl[(blk * D + ch) * 32 + (((t >> 3) ^ swz(ch)) << 3) + (t & 7)] = 0;
        }
    };
    const float sc = p.scale_log2;
    // S^T = K Q^T of the tile in K buffer kl: lane holds keys 32*kt + 16*(r/8) + 8*lg + r%8, query q0 + col
    // MFMA row col of tile kt reads key 32*kt + rho(col), rho swapping bits 2 and 3,
    // so the score registers come out in the order the PV B operand needs.
    const int krho = (col & 19) | ((col & 4) << 1) | ((col & 8) >> 1);
    auto k_at = [&](const uint16_t *kl, int kt, int st) {
        const int slice = st >> 1, c = 2 * (st & 1) + lg;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
            &kl[((kt * NS + slice) * 32 + krho) * 32 + ((c ^ swz(krho)) << 3)]));
    };
    auto qk = [&](const uint16_t *kl, floatx16 (&s)[2]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_at(kl, kt, 0), qb[0], floatx16{}, 0, 0, 0);
#pragma unroll
            for (int st = 1; st < D / 16; ++st)
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_at(kl, kt, st), qb[st], s[kt], 0, 0, 0);
        }
    };
    // online softmax of the scores s (diag: causal mask against key0): rescale
    // O and l when the running max moves, and pack P = exp2(s * sc - m) as the
    // bf16 B operands of the four k-steps of O^T += V^T P^T.  l sums exactly
    // those bf16 values (two per v_dot2_f32_bf16 against (1, 1)), so numerator
    // and denominator carry the same rounding.
    auto softmax_p = [&](floatx16 (&s)[2], int key0, bool diag, bf16x8 (&pb)[4]) {
        if (diag) {
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
        const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                uint32_t pk[4];
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const float e0v = exp2_fast(fmaf(s[kt][8 * st + j], sc, -mb));
                    const float e1v = exp2_fast(fmaf(s[kt][8 * st + j + 1], sc, -mb));
                    const bf16x2 e01 = __builtin_convertvector(floatx2{e0v, e1v}, bf16x2);
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(e01, ones, l_run, false);
                    pk[j / 2] = __builtin_bit_cast(uint32_t, e01);
                }
                pb[2 * kt + st] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            }
    };
    // O^T += V^T P^T over the tile in V buffer vl; k-step (kt, st) covers keys 32*kt + 16*st + 8*lg + j.
    // The A operands of the first k-step come in `first`, read before the
    // barrier that opens the MFMA phase (the tile has long landed), so the
    // phase's first products do not wait for LDS.
    auto v_at = [&](const uint16_t *vl, int kt, int st, int dt) {
        const int ch = 32 * dt + col, c = 2 * st + lg;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&vl[(kt * D + ch) * 32 + ((c ^ swz(ch)) << 3)]));
    };
    auto pv = [&](const uint16_t *vl, const bf16x8 (&pb)[4], const bf16x8 (&first)[4]) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 va = dt == 0 ? first[ks] : v_at(vl, ks >> 1, ks & 1, dt);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], o[dt], 0, 0, 0);
            }
    };

    // s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
    // 11:8), issued through the builtin so the compiler knows what has landed
    constexpr int kWaitVm0 = 0x0F70;                  // vmcnt(0)
    constexpr int kWaitStep = 0x0070 | (2 * KPT);     // vmcnt(2 KPT) lgkmcnt(0): one step's fetches may stay in flight
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    // Every step issues the same two fetches, so the count of loads in flight
    // is the same on every path (the compiler then knows which tiles have
    // landed); past the row's end a step fetches the row's last tile again
    // into a buffer that is not read again.
    auto clamp_tile = [&](int ii) { return tile_of(min(ii, n_iter - 1)); };
    // prologue: K(0), V(0) and K(1) in LDS.  The key tiles of steps ii - 1,
    // ii and ii + 1 travel from step to step: a step looks up only tile ii + 2.
    int c_prev = tile_of(0), c_cur = c_prev, c_n1 = clamp_tile(1);
    size_t base_next = tile_base(tile_id(c_cur));    // pool offset of the tile whose V is fetched next
    fetch(kpool, k_lds0, base_next);
    fetch(vpool, v_lds0, base_next);
    base_next = tile_base(tile_id(c_n1));
    fetch(kpool, k_lds1, base_next);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    floatx16 sa[2], sb[2];                           // scores of even / odd tiles
    auto bar = [] {                                  // a plain barrier, kept in place by the compiler
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // Ping-pong.  A step is a VALU phase (the previous tile's softmax) and an
    // MFMA phase (its PV product, then this tile's QK^T), each closed by a
    // barrier.  Waves 4-7 pass one extra barrier first and so run one phase
    // behind waves 0-3: the two wavefronts of a SIMD (w and w + 4) alternate,
    // one computing exponentials while the other feeds the matrix core.  The
    // ring keeps this safe: a fetch writes a buffer three tiles away from any
    // the other group reads, and every tile has been waited for by both
    // groups before the barrier that opens a phase reading it.
    const bool lag = wave >= 4;
    if (lag) bar();
    auto step = [&](auto b, int ii, floatx16 (&s_cur)[2], floatx16 (&s_prev)[2]) {
        constexpr int B = decltype(b)::value;        // == ii % 4
        using Next2 = std::integral_constant<int, B + 2>;
        using Next1 = std::integral_constant<int, B + 1>;
        using Prev = std::integral_constant<int, B + 3>;
        // K(ii+2) and V(ii+1) land during the step, in buffers last read two
        // steps ago; the V tile's pool offset is the one its K fetch used
        const int c_n2 = clamp_tile(ii + 2);
        const size_t base_k = tile_base(tile_id(c_n2));
        fetch(kpool, kbuf(Next2{}), base_k);
        fetch(vpool, vbuf(Next1{}), base_next);
        base_next = base_k;
        // With QT == 1 every pair has a head (head_ok is false only past the
        // group's last head); with QT > 1 sees() is false for a pair without a
        // query tile.  ii > 0 is known in three of the four unrolled steps.
        const bool prev_ok = (B != 0 || ii > 0) && (QT == 1 ? head_ok : sees(c_prev));
        const bool cur_ok = QT == 1 ? head_ok : sees(c_cur);
        bf16x8 pb[4], vfirst[4];
        if (prev_ok) {
            softmax_p(s_prev, tile_id(c_prev) * kTile, QT > 1 && tile_id(c_prev) == a_s, pb);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) vfirst[ks] = v_at(vbuf(Prev{}), ks >> 1, ks & 1, 0);
        }
        bar();
        if (prev_ok) pv(vbuf(Prev{}), pb, vfirst);
        if (cur_ok) qk(kbuf(b), s_cur);
        // K(ii+1) and V(ii) have landed and this wavefront's LDS reads are
        // done; this step's own fetches may still be in flight
        __builtin_amdgcn_s_waitcnt(kWaitStep);
        bar();
        c_prev = c_cur;
        c_cur = c_n1;
        c_n1 = c_n2;
    };
    for (int ii = 0;; ii += 4) {
        step(I0{}, ii, sa, sb);
        if (ii + 1 >= n_iter) break;
        step(I1{}, ii + 1, sb, sa);
        if (ii + 2 >= n_iter) break;
        step(I2{}, ii + 2, sa, sb);
        if (ii + 3 >= n_iter) break;
        step(I3{}, ii + 3, sb, sa);
        if (ii + 4 >= n_iter) break;
    }
    if (!lag) bar();                                 // the groups meet again
    // epilogue: the last tile (the diagonal one of the highest query tile);
    // its values past T may hold any bits: zero them, so a zero probability
    // never meets a NaN
    const int c_last = c_prev;                       // tile n_iter - 1
    const int lb = (n_iter - 1) & 3;
    uint16_t *vl_last = lb == 0 ? v_lds0 : lb == 1 ? v_lds1 : lb == 2 ? v_lds2 : v_lds3;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);            // no fetch lands after this point
    __syncthreads();
    zero_v_tail(vl_last, tile_id(c_last) * kTile);
    __syncthreads();
    if (head_ok && (QT == 1 || sees(c_last))) {
        const bool diag = QT == 1 || tile_id(c_last) == a_s;
        bf16x8 pb[4], vfirst[4];
        if ((n_iter - 1) & 1) softmax_p(sb, tile_id(c_last) * kTile, diag, pb);
        else softmax_p(sa, tile_id(c_last) * kTile, diag, pb);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vfirst[ks] = v_at(vl_last, ks >> 1, ks & 1, 0);
        pv(vl_last, pb, vfirst);
    }

    if (p.tile_counter) {
        if constexpr (QT == 1) {
            if (tid == 0) {
                const int heads_here = min(4, G - it.hg * 4);
                atomicAdd(p.tile_counter, (unsigned long long)n_iter * heads_here);
            }
        } else if (head_ok && (wave & 1) == 0 && lane == 0) {
            // the tiles this pair's query tile sees
            if constexpr (kUnion) {
                const int32_t *rp = p.row_ptr + (size_t)it.kv * (p.n_qblocks + 1) + a_s;
                const int b0 = min(max(rp[0], 0), p.nnz);
                atomicAdd(p.tile_counter, (unsigned long long)(min(max(rp[1], b0), p.nnz) - b0));
            } else {
                const int e0s = it.streaming ? min(p.sink_blocks, a_s + 1) : 0;
                const int s1s = it.streaming ? max(a_s - p.local_blocks + 1, e0s) : 0;
                atomicAdd(p.tile_counter, (unsigned long long)(e0s + (a_s - s1s + 1)));
            }
        }
    }
    if (!head_ok) return;
    // ---- normalise and store: lane holds query q0 + col, channels 32*dt + 8*(r/4) + 4*lg + r%4
    const float lt = sum_xor32(l_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;    // a query tile whose own row is empty: zero output
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
template <int D, bool CSR>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs p) {
    extern __shared__ float sm[];
    float *k_lds = sm;                 // [64][D]
    float *v_lds = sm + kTile * D;     // [D][64]

    const PItem it = prefill_item<CSR, 1>(p);
    const TileRow trow = tile_row<CSR, 1>(p, it);

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
    const int n_iter = trow.n;
    for (int ii = 0; ii < n_iter; ++ii) {
        const int c = row_tile<CSR>(p, it, trow, ii);
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
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;      // no visible key: zero output
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
}

}  // namespace

template <int D, bool CSR>
void launch_bf16(const PrefillArgs &p, dim3 grid, hipStream_t s) {
    if (p.q_tiles == 1) hipLaunchKernelGGL((prefill_bf16_kernel<D, CSR, 1>), grid, dim3(512), 0, s, p);
    else if (p.q_tiles == 2) hipLaunchKernelGGL((prefill_bf16_kernel<D, CSR, 2>), grid, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((prefill_bf16_kernel<D, CSR, 4>), grid, dim3(512), 0, s, p);
}

template <bool CSR>
void launch_prefill_kernels(const PrefillArgs &p, int dtype, hipStream_t s) {
    const dim3 grid((unsigned)p.n_items);
    if (dtype == LSA_BF16) {
        if (p.head_dim == 128) launch_bf16<128, CSR>(p, grid, s);
        else launch_bf16<64, CSR>(p, grid, s);
    } else {
        // f32 is the small-model path: head_dim 64 only (validated by the caller)
        const size_t lds = 2 * (size_t)kTile * 64 * sizeof(float);
        hipLaunchKernelGGL((prefill_f32_kernel<64, CSR>), grid, dim3(256), lds, s, p);
    }
}

hipError_t launch_prefill(const PrefillArgs &p, int dtype, hipStream_t s) {
    if (p.n_items == 0) return hipSuccess;
    if (p.row_ptr) launch_prefill_kernels<true>(p, dtype, s);
    else launch_prefill_kernels<false>(p, dtype, s);
    return hipGetLastError();
}

}  // namespace lsa
