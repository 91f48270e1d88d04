// Logical-page key statistics: channel-wise min and max of the keys of each
// N_L-token logical page (LServe explainer, 技術的詳細 / 動的スパーシティ:
// k_min^j and k_max^j per channel; 階層的ページング: logical pages inside
// N_P-token physical pages, kept beside the physical page).
//
// One wavefront per (sequence, KV head, logical page).  Each lane owns one or
// two adjacent channels and walks the page's valid rows (a row of the key
// tiles is 32 channels, so a wavefront's read of one token is D/32 runs of 32
// channels).  Min / max select one of the inputs, so the results are exact in
// the storage type.
#include "lsa_internal.h"

namespace lsa {
namespace {

struct Item {
    int b, kv, m, jl, row0, rows, pool;
    bool valid;
};

__device__ __forceinline__ Item locate(const StatsArgs &a) {
    Item it;
    const int wave = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int total = a.batch * a.n_heads_sel * a.lp_per_seq;
    it.valid = wave < total;
    if (!it.valid) return it;
    const int jj = wave % a.lp_per_seq;
    const int rest = wave / a.lp_per_seq;
    const int hi = rest % a.n_heads_sel;
    it.b = rest / a.n_heads_sel;
    it.kv = a.heads_sel[hi];
    const int L = a.seq_lens[it.b];
    const int first = a.first_token ? a.first_token[it.b] : 0;
    const int j = first / a.logical_page + jj;
    const int t0 = j * a.logical_page;
    if (t0 >= L || first < 0) { it.valid = false; return it; }
    const int g = a.page_size / a.logical_page;
    it.m = j / g;
    it.jl = j % g;
    it.row0 = it.jl * a.logical_page;
    it.rows = min(a.logical_page, L - t0);
    it.pool = a.page_table[(size_t)it.b * a.max_pages + it.m];
    return it;
}

// f32 / bf16 keys.  CPL = channels per lane (D / 64).
template <typename Elem, int CPL>
__global__ __launch_bounds__(256) void stats_float_kernel(StatsArgs a) {
    const Item it = locate(a);
    if (!it.valid) return;
    const int lane = threadIdx.x % kWave;
    const int D = a.head_dim;
    const int g = a.page_size / a.logical_page;
    const size_t page_base = ((size_t)it.pool * a.hm.pool_heads + pool_slot(a.hm, it.kv)) * a.page_size * D;
    const Elem *k = static_cast<const Elem *>(a.k);
    float mn[CPL], mx[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) { mn[c] = __builtin_inff(); mx[c] = -__builtin_inff(); }
    for (int r = 0; r < it.rows; ++r) {
        const Elem *row = k + page_base + key_offset(it.row0 + r, lane * CPL, D, block_shift(a.page_size));
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float x;
            if constexpr (sizeof(Elem) == 2) x = bf16_to_f32(row[c]);
            else x = row[c];
            mn[c] = fminf(mn[c], x);
            mx[c] = fmaxf(mx[c], x);
        }
    }
    Elem *out = static_cast<Elem *>(a.stats) +
                ((((size_t)it.pool * a.hm.pool_heads + pool_slot(a.hm, it.kv)) * g + it.jl) * 2) * D + lane * CPL;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if constexpr (sizeof(Elem) == 2) {
            out[c] = uint16_t(__float_as_uint(mn[c]) >> 16);      // exact: mn is a bf16 value
            out[D + c] = uint16_t(__float_as_uint(mx[c]) >> 16);
        } else {
            out[c] = mn[c];
            out[D + c] = mx[c];
        }
    }
}

// int4 keys: a tile row's byte i holds channels 2i (low nibble) and 2i+1.
// Output byte per channel: c_min | c_max << 4.
__global__ __launch_bounds__(256) void stats_int4_kernel(StatsArgs a) {
    const Item it = locate(a);
    if (!it.valid) return;
    const int lane = threadIdx.x % kWave;
    const int D = a.head_dim;
    const int row_bytes = D / 2;
    if (lane >= row_bytes) return;
    const int g = a.page_size / a.logical_page;
    const size_t page_base = ((size_t)it.pool * a.hm.pool_heads + pool_slot(a.hm, it.kv)) * a.page_size * D;
    const uint8_t *k = static_cast<const uint8_t *>(a.k);
    uint32_t lo_min = 15, lo_max = 0, hi_min = 15, hi_max = 0;
    for (int r = 0; r < it.rows; ++r) {
        const uint32_t byte = k[(page_base + key_offset(it.row0 + r, 2 * lane, D, block_shift(a.page_size))) / 2];
        const uint32_t lo = byte & 15u, hi = byte >> 4;
        lo_min = min(lo_min, lo); lo_max = max(lo_max, lo);
        hi_min = min(hi_min, hi); hi_max = max(hi_max, hi);
    }
    uint8_t *out = static_cast<uint8_t *>(a.stats) +
                   (((size_t)it.pool * a.hm.pool_heads + pool_slot(a.hm, it.kv)) * g + it.jl) * D + 2 * lane;
    const uint16_t pair = uint16_t((lo_min | (lo_max << 4)) | ((hi_min | (hi_max << 4)) << 8));
    *reinterpret_cast<uint16_t *>(out) = pair;
}

}  // namespace

hipError_t launch_stats(const StatsArgs &a, hipStream_t s) {
    const long long waves = (long long)a.batch * a.n_heads_sel * a.lp_per_seq;
    if (waves == 0) return hipSuccess;
    const int wpb = 4;
    const unsigned grid = (unsigned)((waves + wpb - 1) / wpb);
    if (a.dtype == LSA_INT4) {
        hipLaunchKernelGGL(stats_int4_kernel, dim3(grid), dim3(256), 0, s, a);
    } else if (a.dtype == LSA_BF16) {
        if (a.head_dim == 128) hipLaunchKernelGGL((stats_float_kernel<uint16_t, 2>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((stats_float_kernel<uint16_t, 1>), dim3(grid), dim3(256), 0, s, a);
    } else {
        if (a.head_dim == 128) hipLaunchKernelGGL((stats_float_kernel<float, 2>), dim3(grid), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((stats_float_kernel<float, 1>), dim3(grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace lsa
