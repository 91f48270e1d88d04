// Appending the newest token's key and value, and filling the constant-size
// cache of the streaming heads (LServe explainer, 技術的詳細 / 静的スパーシティ:
// a streaming head only attends its sink and its most recent tokens, so it
// needs a cache of constant size; Reusable Page Selection: a decode step
// appends its token's K/V before the selection and the attention).
//
// Append: one wavefront per (sequence, KV head); lanes own channels.  The key
// goes to row t % N_P of the page's key tiles, the value to column t % N_P of
// its value rows (int4: the token's nibble of each value byte is replaced,
// keeping the neighbouring token's).  For retrieval heads the statistics of
// the logical page that holds t take the token in: a logical page that t
// opens starts from it, otherwise min / max fold it in (exact, no rounding).
//
// Fill: one workgroup per (sequence, streaming head, cache page) copies the
// whole pool page that the cache page stands for.
#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kAppendWaves = 4;

template <int KV_DT>
__global__ __launch_bounds__(kAppendWaves * kWave) void append_kernel(AppendArgs a) {
    const int item = blockIdx.x * kAppendWaves + threadIdx.x / kWave;
    if (item >= a.batch * a.num_kv_heads) return;
    const int lane = threadIdx.x % kWave;
    const int b = item / a.num_kv_heads, kv = item % a.num_kv_heads;
    const int D = a.head_dim, NP = a.page_size, NL = a.logical_page;
    const int bs = block_shift(NP);
    const int t = a.seq_lens[b] - 1;
    const int m = t / NP, slot = t % NP;
    const bool streaming = head_streaming(a.hm, kv);
    const bool in_cache = streaming && a.sc_k != nullptr;
    const size_t hp = in_cache ? (size_t)stream_cache_page(b, streaming_rank(a.hm, kv), m, a.n_str, a.sc_sink, a.sc_ring)
                               : (size_t)a.page_table[(size_t)b * a.max_pages + m] * a.hm.pool_heads +
                                     pool_slot(a.hm, kv);
    const size_t page_base = hp * NP * D;
    const size_t row = (size_t)item * D;          // the token's K / V row in k_new, v_new
    const bool upd = a.stats != nullptr && !streaming;
    const int g = NP / NL, jl = slot / NL;
    const bool opens = slot % NL == 0;            // t is the first token of its logical page
    if constexpr (KV_DT == LSA_INT4) {
        uint8_t *kd = static_cast<uint8_t *>(in_cache ? a.sc_k : a.k);
        uint8_t *vd = static_cast<uint8_t *>(in_cache ? a.sc_v : a.v);
        const uint8_t *kn = static_cast<const uint8_t *>(a.k_new);
        const uint8_t *vn = static_cast<const uint8_t *>(a.v_new);
        if (lane < D / 2) {
            // byte `lane` of the row: channels 2 * lane (low nibble) and 2 * lane + 1
            const uint32_t kb = kn[row / 2 + lane];
            kd[(page_base + key_offset(slot, 2 * lane, D, bs)) / 2] = (uint8_t)kb;
            const uint32_t vb = vn[row / 2 + lane];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t code = (vb >> (4 * e)) & 15u;
                uint8_t *p = vd + (page_base + value_offset(slot, 2 * lane + e, D, bs)) / 2;
                const uint32_t old = *p;
                *p = (uint8_t)((slot & 1) ? ((old & 0x0Fu) | (code << 4)) : ((old & 0xF0u) | code));
            }
            if (upd) {
                // statistics byte per channel: c_min | c_max << 4
                uint8_t *st = static_cast<uint8_t *>(a.stats) + (hp * g + jl) * D + 2 * lane;
                const uint32_t prev = opens ? 0u : *reinterpret_cast<const uint16_t *>(st);
                uint32_t out = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t c = (kb >> (4 * e)) & 15u;
                    const uint32_t pb = (prev >> (8 * e)) & 0xFFu;
                    const uint32_t mn = opens ? c : min(pb & 15u, c);
                    const uint32_t mx = opens ? c : max(pb >> 4, c);
                    out |= (mn | (mx << 4)) << (8 * e);
                }
                *reinterpret_cast<uint16_t *>(st) = (uint16_t)out;
            }
        }
        if (lane == 0) {
            uint16_t *ks = in_cache ? a.sc_k_sz : a.k_sz;
            uint16_t *vs = in_cache ? a.sc_v_sz : a.v_sz;
            *reinterpret_cast<uint32_t *>(ks + hp * 2) = *reinterpret_cast<const uint32_t *>(a.k_new_sz + (size_t)item * 2);
            *reinterpret_cast<uint32_t *>(vs + hp * 2) = *reinterpret_cast<const uint32_t *>(a.v_new_sz + (size_t)item * 2);
        }
    } else {
        using Elem = typename std::conditional<KV_DT == LSA_F32, float, uint16_t>::type;
        Elem *kd = static_cast<Elem *>(in_cache ? a.sc_k : a.k);
        Elem *vd = static_cast<Elem *>(in_cache ? a.sc_v : a.v);
        const Elem *kn = static_cast<const Elem *>(a.k_new);
        const Elem *vn = static_cast<const Elem *>(a.v_new);
        for (int c = lane; c < D; c += kWave) {
            const Elem kx = kn[row + c];
            kd[page_base + key_offset(slot, c, D, bs)] = kx;
            vd[page_base + value_offset(slot, c, D, bs)] = vn[row + c];
            if (upd) {
                Elem *st = static_cast<Elem *>(a.stats) + ((hp * g + jl) * 2) * D + c;
                float x, lo, hi;
                if constexpr (KV_DT == LSA_F32) {
                    x = kx; lo = st[0]; hi = st[D];
                } else {
                    x = bf16_to_f32(kx); lo = bf16_to_f32(st[0]); hi = bf16_to_f32(st[D]);
                }
                const float mn = opens ? x : fminf(lo, x);
                const float mx = opens ? x : fmaxf(hi, x);
                if constexpr (KV_DT == LSA_F32) {
                    st[0] = mn;
                    st[D] = mx;
                } else {                                   // exact: mn, mx are bf16 values
                    st[0] = uint16_t(__float_as_uint(mn) >> 16);
                    st[D] = uint16_t(__float_as_uint(mx) >> 16);
                }
            }
        }
    }
}

constexpr int kFillThreads = 256;

__global__ __launch_bounds__(kFillThreads) void stream_fill_kernel(FillArgs a) {
    const int per = a.sc_sink + a.sc_ring;
    const int cp = blockIdx.x % per;
    const int rest = blockIdx.x / per;
    const int s = rest % a.n_str;
    const int b = rest / a.n_str;
    const int L = a.seq_lens[b];
    if (L <= 0) return;
    const int m_cur = (L - 1) / a.page_size;
    int m;
    if (cp < a.sc_sink) {
        m = cp;
        if (m > m_cur) return;
    } else {
        // the most recent page m >= sink whose ring slot is cp - sink
        const int r = cp - a.sc_sink, top = m_cur - a.sc_sink;
        if (top < 0) return;
        const int mm = top - ((top - r) % a.sc_ring + a.sc_ring) % a.sc_ring;
        if (mm < 0) return;
        m = a.sc_sink + mm;
    }
    const int kv = a.str_heads[s];
    const size_t src = (size_t)a.page_table[(size_t)b * a.max_pages + m] * a.num_kv_heads + kv;
    const size_t dst = blockIdx.x;                // the cache page (b, s, cp)
    const size_t elems = (size_t)a.page_size * a.head_dim;
    const size_t bytes = a.dtype == LSA_F32 ? elems * 4 : a.dtype == LSA_BF16 ? elems * 2 : elems / 2;
    const uint4 *ks = reinterpret_cast<const uint4 *>(static_cast<const char *>(a.k) + src * bytes);
    const uint4 *vs = reinterpret_cast<const uint4 *>(static_cast<const char *>(a.v) + src * bytes);
    uint4 *kd = reinterpret_cast<uint4 *>(static_cast<char *>(a.sc_k) + dst * bytes);
    uint4 *vd = reinterpret_cast<uint4 *>(static_cast<char *>(a.sc_v) + dst * bytes);
    for (size_t i = threadIdx.x; i < bytes / 16; i += kFillThreads) {
        kd[i] = ks[i];
        vd[i] = vs[i];
    }
    if (a.dtype == LSA_INT4 && threadIdx.x == 0) {
        *reinterpret_cast<uint32_t *>(a.sc_k_sz + dst * 2) = *reinterpret_cast<const uint32_t *>(a.k_sz + src * 2);
        *reinterpret_cast<uint32_t *>(a.sc_v_sz + dst * 2) = *reinterpret_cast<const uint32_t *>(a.v_sz + src * 2);
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
    const long long items = (long long)a.batch * a.num_kv_heads;
    if (items == 0) return hipSuccess;
    const dim3 grid((unsigned)((items + kAppendWaves - 1) / kAppendWaves)), block(kAppendWaves * kWave);
    if (a.dtype == LSA_INT4) hipLaunchKernelGGL(append_kernel<LSA_INT4>, grid, block, 0, s, a);
    else if (a.dtype == LSA_BF16) hipLaunchKernelGGL(append_kernel<LSA_BF16>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(append_kernel<LSA_F32>, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_stream_fill(const FillArgs &a, hipStream_t s) {
    const long long grid = (long long)a.batch * a.n_str * (a.sc_sink + a.sc_ring);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(stream_fill_kernel, dim3((unsigned)grid), dim3(kFillThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace lsa
