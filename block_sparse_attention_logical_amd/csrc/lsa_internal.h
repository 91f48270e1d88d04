// Internal declarations shared by the HIP translation units of liblsa.
// Not part of the public ABI (include/lsa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa.h"

namespace lsa {

constexpr int kMaxKvHeads = 64;   // H_kv limit (host-side tables live in kernel args)
constexpr int kWave = 64;         // CDNA wavefront width
constexpr int kMaxDecodeChunks = 128;   // split-KV chunks per (sequence, KV head)

// ----------------------------------------------------------------------------
// numeric helpers (device)
// ----------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite here)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// IEEE binary16 bits -> float (exact)
__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return float(v);
}

// 2^x on the hardware exponential unit
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------------------------
// launch arguments
// ----------------------------------------------------------------------------

struct StatsArgs {
    const void *k;
    const uint16_t *k_sz;
    void *stats;
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *first_token;   // may be null
    int32_t batch, max_pages, num_kv_heads, head_dim, page_size, logical_page;
    int32_t n_heads_sel;          // number of KV heads processed
    int32_t lp_per_seq;           // logical pages covered per (sequence, head)
    int32_t dtype;
    uint8_t heads_sel[kMaxKvHeads];
};

struct ScoreArgs {
    const void *q;
    const void *stats;
    const void *k;                // the key pool: the current logical page is scored from its keys
    const uint16_t *k_sz;
    const int32_t *page_table;
    const int32_t *seq_lens;
    double *phys;                 // [B][H_kv][max_pages]
    int32_t batch, max_pages, num_q_heads, num_kv_heads, head_dim, page_size, logical_page;
    int32_t q_dtype, kv_dtype;
    int32_t n_ret;                // number of retrieval heads
    int32_t pages_per_block;      // physical pages per workgroup
    int32_t blocks_per_head;      // workgroups per (sequence, retrieval head)
    uint8_t ret_heads[kMaxKvHeads];
};

struct TopkArgs {
    const double *phys;
    const int32_t *seq_lens;
    int32_t *selected;            // [B][H_kv][K]
    int32_t batch, max_pages, num_kv_heads, page_size, k;
    int32_t n_ret;
    uint8_t ret_heads[kMaxKvHeads];
};

struct DecodeArgs {
    const void *q;
    void *out;
    const void *k;
    const void *v;
    const uint16_t *k_sz;
    const uint16_t *v_sz;
    const int32_t *page_table;
    const int32_t *seq_lens;
    const int32_t *selected;
    float *part;                  // partial records
    void *stats;                  // may be null: refresh the current logical page's statistics
    int32_t batch, max_pages, num_q_heads, num_kv_heads, group, head_dim, page_size, logical_page;
    int32_t sel_k;                // K (row length of selected)
    int32_t sink, local;
    int32_t chunks_ret, chunks_str;   // workgroups per (sequence, head) by kind
    int32_t chunks_max;               // record slots per (sequence, head)
    int32_t chunks_per_seq;           // workgroups per sequence
    int32_t pages_per_wave;
    float scale_log2;                 // softmax scale * log2(e)
    uint8_t kind[kMaxKvHeads];
};

struct PrefillArgs {
    const void *q;
    void *out;
    const void *k;
    const void *v;
    const int32_t *page_table;
    unsigned long long *tile_counter;
    int32_t seq_len, num_q_heads, num_kv_heads, group, head_dim, page_size;
    int32_t sink_blocks, local_blocks;
    int32_t n_qblocks;
    int32_t n_items;              // work items (kv head, query tile, head group)
    int32_t head_groups;          // query-head groups of 4 per KV head
    float scale_log2;
    int32_t n_ret, n_str;         // retrieval / streaming KV heads
    uint8_t ret_heads[kMaxKvHeads];
    uint8_t str_heads[kMaxKvHeads];
};

// ----------------------------------------------------------------------------
// launchers (each returns hipSuccess or the launch error)
// ----------------------------------------------------------------------------

hipError_t launch_stats(const StatsArgs &a, hipStream_t s);
hipError_t launch_score(const ScoreArgs &a, hipStream_t s);
int score_pages_per_block(int kv_dtype, int head_dim, int page_size, int logical_page);
int topk_max_pages();
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int q_dtype, int kv_dtype, hipStream_t s);
hipError_t launch_combine(const DecodeArgs &a, int q_dtype, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t s);

}  // namespace lsa
