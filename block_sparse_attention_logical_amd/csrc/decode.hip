// Block-sparse paged decode attention for retrieval and streaming heads
// (LServe explainer, 技術的詳細 / 静的スパーシティ: streaming heads see the sink
// and the recent tokens; 動的スパーシティ and the figure: retrieval heads read
// only their top-K physical pages; 統一ブロックスパースアテンション: one
// block-sparse kernel serves both head kinds; abstract page: a constant number
// of KV pages per step).
//
// Work decomposition (split-KV).  The attended page list of a (sequence, KV
// head) is cut into chunks of 4 * pages_per_wave pages; one workgroup of four
// wavefronts takes a chunk, each wavefront streams its pages with an online
// softmax, the four states are merged in LDS and one partial record
// (max, sum, unnormalised output) is written per chunk.  A second, small
// kernel merges the records of each (sequence, KV head) in chunk order, so
// results are deterministic.  Every K/V page read serves all G query heads of the
// group.
//
// bf16 path: both contractions run on v_mfma_f32_16x16x32_bf16 straight from
// registers.  QK^T is computed transposed (tokens in M, heads in N), so a lane
// loads 16 contiguous bytes of one key row; the 32 keys of a block are
// assigned to MFMA rows so that the score tile a lane receives is exactly the
// B operand the PV product needs (8 consecutive tokens of one head), and the
// V page is stored channel-major so the A operand of PV (one channel, 8
// consecutive tokens) is again one 16-byte load.  Heads occupy the N
// dimension, padded to 16 with zero queries.
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
    w.L = a.seq_lens[w.b];
    w.t = w.L - 1;
    w.streaming = a.kind[kv] != 0;
    return w;
}

// The attended physical pages of one (sequence, KV head), in ascending order.
struct PageList {
    int n;                 // list length
    // retrieval
    const int32_t *sel;
    int n_sel, cur;
    bool cur_in;
    // streaming
    int n_sink_pages, local_first;

    __device__ __forceinline__ int page(int i) const {
        if (sel) return i < n_sel ? sel[i] : cur;
        return i < n_sink_pages ? i : local_first + (i - n_sink_pages);
    }
};

__device__ __forceinline__ PageList make_list(const DecodeArgs &a, const WorkItem &w) {
    PageList pl;
    const int NP = a.page_size;
    pl.cur = w.t / NP;
    if (w.streaming) {
        pl.sel = nullptr;
        pl.n_sel = 0;
        pl.cur_in = false;
        const int sink_end = min(a.sink, w.t + 1);            // tokens [0, sink_end)
        pl.n_sink_pages = (sink_end + NP - 1) / NP;
        const int lf = max(0, w.t - a.local + 1) / NP;         // first local page
        pl.local_first = max(lf, pl.n_sink_pages);
        pl.n = pl.n_sink_pages + max(0, pl.cur - pl.local_first + 1);
    } else {
        pl.sel = a.selected + ((size_t)w.b * a.num_kv_heads + w.kv) * a.sel_k;
        const int lane = threadIdx.x % kWave;
        int cnt = 0;
        bool in = false;
        for (int i0 = 0; i0 < a.sel_k; i0 += kWave) {
            const int i = i0 + lane;
            const int m = i < a.sel_k ? pl.sel[i] : -1;
            cnt += __popcll(__ballot(m >= 0));
            in |= __ballot(m == pl.cur) != 0;
        }
        pl.n_sel = cnt;
        pl.cur_in = in;
        pl.n_sink_pages = 0;
        pl.local_first = 0;
        pl.n = cnt + (in ? 0 : 1);
    }
    return pl;
}

__device__ __forceinline__ bool token_visible(const DecodeArgs &a, const WorkItem &w, int p) {
    if (p > w.t) return false;
    if (!w.streaming) return true;
    return p < a.sink || (w.t - p) < a.local;
}

// Merge the per-wave softmax states held in LDS and write this chunk's record.
// LDS layout per wave: m[16], l[16], o[16][D].
__device__ __forceinline__ void merge_waves_and_store(const DecodeArgs &a, const WorkItem &w,
                                                      const float *lds, int D) {
    const int G = a.group;
    const int wave_stride = 32 + 16 * D;
    const size_t rec_size = 32 + (size_t)G * D;
    float *rec = a.part + (((size_t)w.b * a.num_kv_heads + w.kv) * a.chunks_max + w.chunk) * rec_size;
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D, d = idx % D;
        float M = -__builtin_inff();
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, lds[wv * wave_stride + h]);
        float acc = 0.f, lsum = 0.f;
        if (M != -__builtin_inff()) {
#pragma unroll
            for (int wv = 0; wv < 4; ++wv) {
                const float mw = lds[wv * wave_stride + h];
                const float wt = mw == -__builtin_inff() ? 0.f : exp2_fast(mw - M);
                acc += wt * lds[wv * wave_stride + 32 + h * D + d];
                lsum += wt * lds[wv * wave_stride + 16 + h];
            }
        }
        rec[32 + idx] = acc;
        if (d == 0) {
            rec[h] = M;
            rec[16 + h] = lsum;
        }
    }
}

// ---------------------------------------------------------------------------
// split-KV combine (a second kernel: the kernel boundary orders the records,
// so no device-scope fence, which would write back and invalidate the whole
// L2 of the XCD, is needed)
// ---------------------------------------------------------------------------
// Merge the chunk records of (b, kv) in chunk order (deterministic) and write
// the normalised output in q's dtype.
template <typename OutT>
__device__ __forceinline__ void combine_records(const DecodeArgs &a, int b, int kv) {
    const int G = a.group, D = a.head_dim;
    const int nchunks = a.kind[kv] ? a.chunks_str : a.chunks_ret;
    const size_t rec_size = 32 + (size_t)G * D;
    const float *rec0 = a.part + ((size_t)b * a.num_kv_heads + kv) * a.chunks_max * rec_size;
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D;
        float M = -__builtin_inff();
        for (int c = 0; c < nchunks; ++c) M = fmaxf(M, rec0[c * rec_size + h]);
        float acc = 0.f, lsum = 0.f;
        for (int c = 0; c < nchunks; ++c) {
            const float *rec = rec0 + c * rec_size;
            const float mc = rec[h];
            if (mc == -__builtin_inff()) continue;
            const float wt = exp2_fast(mc - M);
            acc += wt * rec[32 + idx];
            lsum += wt * rec[16 + h];
        }
        const float val = acc / lsum;
        const size_t o = ((size_t)b * a.num_q_heads + (size_t)kv * G) * D + idx;
        if constexpr (sizeof(OutT) == 2) static_cast<uint16_t *>(a.out)[o] = f32_to_bf16_rne(val);
        else static_cast<float *>(a.out)[o] = val;
    }
}

// ---------------------------------------------------------------------------
// bf16 K/V, bf16 q: MFMA path
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeArgs a) {
    extern __shared__ float lds[];
    const WorkItem w = decode_item(a);
    const PageList pl = make_list(a, w);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int h = lane & 15, g4 = lane >> 4;
    const int G = a.group, NP = a.page_size;

    // B operand of QK^T: column h = query head, k = channel s*32 + 8*g4 + j
    bf16x8 qb[D / 32];
    {
        const uint16_t *q = static_cast<const uint16_t *>(a.q) +
                            ((size_t)w.b * a.num_q_heads + (size_t)w.kv * G + min(h, G - 1)) * D;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            uint4 raw = *reinterpret_cast<const uint4 *>(q + s * 32 + 8 * g4);
            if (h >= G) raw = make_uint4(0, 0, 0, 0);
            qb[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    floatx4 o[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff(), l_run = 0.f;

    const int ppw = a.pages_per_wave;
    const int i_begin = w.chunk * 4 * ppw + wave * ppw;
    const int i_end = min(i_begin + ppw, pl.n);
    const uint16_t *kpool = static_cast<const uint16_t *>(a.k);
    const uint16_t *vpool = static_cast<const uint16_t *>(a.v);

    for (int i = i_begin; i < i_end; ++i) {
        const int page = pl.page(i);
        const int pool = a.page_table[(size_t)w.b * a.max_pages + page];
        const size_t head_page = (size_t)pool * a.num_kv_heads + w.kv;
        const uint16_t *kb_ptr = kpool + head_page * NP * D;
        const uint16_t *vb_ptr = vpool + head_page * D * NP;
        const int p0 = page * NP;
        for (int kb = 0; kb < NP / 32; ++kb) {
            const int tok0 = p0 + 32 * kb;
            if (tok0 > w.t) break;
            if (w.streaming) {
                const int p_last = min(tok0 + 31, w.t);
                if (!(tok0 < a.sink || (w.t - p_last) < a.local)) continue;
            }
            // ---- QK^T for the 32 keys of this block (two 16-row tiles)
            // tile T, MFMA row rho -> key 8*(rho/4) + 4*T + rho%4 of the block
            const int rho = lane & 15;
            const int key0 = 32 * kb + 8 * (rho >> 2) + (rho & 3);
            floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                const uint4 r0 = *reinterpret_cast<const uint4 *>(kb_ptr + (size_t)key0 * D + s * 32 + 8 * g4);
                const uint4 r1 = *reinterpret_cast<const uint4 *>(kb_ptr + (size_t)(key0 + 4) * D + s * 32 + 8 * g4);
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r0), qb[s], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r1), qb[s], s1, 0, 0, 0);
            }
            // V^T loads for this block are independent of the softmax: issue them now
            uint4 vr[D / 16];
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                vr[dt] = *reinterpret_cast<const uint4 *>(vb_ptr + (size_t)(16 * dt + h) * NP + 32 * kb + 8 * g4);
            if (tok0 + 31 > w.t) {
                // slots after the current token may hold any bits: zero them so that
                // a zero probability never meets a NaN in the PV product
                const int nvalid = w.t - (tok0 + 8 * g4) + 1;
                uint32_t keep[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    keep[e] = (2 * e < nvalid ? 0x0000FFFFu : 0u) | (2 * e + 1 < nvalid ? 0xFFFF0000u : 0u);
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) {
                    vr[dt].x &= keep[0]; vr[dt].y &= keep[1]; vr[dt].z &= keep[2]; vr[dt].w &= keep[3];
                }
            }
            // lane holds the logits of head h for keys 8*g4 + j, j = 0..7 of the block
            float x[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) { x[r] = s0[r] * a.scale_log2; x[4 + r] = s1[r] * a.scale_log2; }
            float mb = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (!token_visible(a, w, tok0 + 8 * g4 + j)) x[j] = -__builtin_inff();
                mb = fmaxf(mb, x[j]);
            }
            mb = fmaxf(mb, __shfl_xor(mb, 16, kWave));
            mb = fmaxf(mb, __shfl_xor(mb, 32, kWave));
            const float m_new = fmaxf(m_run, mb);
            const float alpha = exp2_fast(m_run - m_new);
            float psum = 0.f;
            uint32_t pk[4];
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const float pa = exp2_fast(x[j] - m_new);
                const float pb = exp2_fast(x[j + 1] - m_new);
                psum += pa + pb;
                pk[j / 2] = uint32_t(f32_to_bf16_rne(pa)) | (uint32_t(f32_to_bf16_rne(pb)) << 16);
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            const bf16x8 pbv = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                o[dt] *= alpha;
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vr[dt]), pbv, o[dt], 0, 0, 0);
            }
        }
    }
    l_run += __shfl_xor(l_run, 16, kWave);
    l_run += __shfl_xor(l_run, 32, kWave);

    float *my = lds + wave * (32 + 16 * D);
    if (g4 == 0) { my[h] = m_run; my[16 + h] = l_run; }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) my[32 + h * D + 16 * dt + 4 * g4 + r] = o[dt][r];
    __syncthreads();
    merge_waves_and_store(a, w, lds, D);
}

// ---------------------------------------------------------------------------
// f32 K/V, f32 q: plain VALU path (lanes own tokens for QK^T, channels for PV)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeArgs a) {
    extern __shared__ float lds[];
    const WorkItem w = decode_item(a);
    const PageList pl = make_list(a, w);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int G = a.group, NP = a.page_size;
    constexpr int CPL = D / 64;                   // channels per lane in PV

    float *qs = lds + 4 * (32 + 16 * D);          // [G][D]
    float *ps = qs + 16 * D + wave * 16 * 64;     // this wave's [16][64] probabilities
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x)
        qs[idx] = static_cast<const float *>(a.q)[((size_t)w.b * a.num_q_heads + (size_t)w.kv * G) * D + idx];
    __syncthreads();

    float o[16][CPL];
    float m_run[16], l_run[16];
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) {
        m_run[hh] = -__builtin_inff();
        l_run[hh] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[hh][c] = 0.f;
    }

    const int ppw = a.pages_per_wave;
    const int i_begin = w.chunk * 4 * ppw + wave * ppw;
    const int i_end = min(i_begin + ppw, pl.n);
    const float *kpool = static_cast<const float *>(a.k);
    const float *vpool = static_cast<const float *>(a.v);

    for (int i = i_begin; i < i_end; ++i) {
        const int page = pl.page(i);
        const int pool = a.page_table[(size_t)w.b * a.max_pages + page];
        const size_t head_page = (size_t)pool * a.num_kv_heads + w.kv;
        const float *kp = kpool + head_page * NP * D;
        const float *vp = vpool + head_page * D * NP;
        for (int s0 = 0; s0 < NP; s0 += kWave) {
            const int slot = s0 + lane;
            const int p = page * NP + slot;
            const bool vis = slot < NP && token_visible(a, w, p);
            float sc[16];
#pragma unroll
            for (int hh = 0; hh < 16; ++hh) sc[hh] = 0.f;
            if (slot < NP) {
                const float *krow = kp + (size_t)slot * D;
                for (int d = 0; d < D; d += 4) {
                    const float4 kv4 = *reinterpret_cast<const float4 *>(krow + d);
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
                float mb = x;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) mb = fmaxf(mb, __shfl_xor(mb, off, kWave));
                if (mb == -__builtin_inff()) { alpha[hh] = 1.f; ps[hh * 64 + lane] = 0.f; continue; }
                const float m_new = fmaxf(m_run[hh], mb);
                alpha[hh] = exp2_fast(m_run[hh] - m_new);
                const float pr = vis ? exp2_fast(x - m_new) : 0.f;
                float psum = pr;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) psum += __shfl_xor(psum, off, kWave);
                l_run[hh] = l_run[hh] * alpha[hh] + psum;
                m_run[hh] = m_new;
                ps[hh * 64 + lane] = pr;
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int nslots = max(0, min(min(kWave, NP - s0), w.t - (page * NP + s0) + 1));
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int d = lane * CPL + c;
                const float *vrow = vp + (size_t)d * NP + s0;
                float acc[16];
#pragma unroll
                for (int hh = 0; hh < 16; ++hh) acc[hh] = o[hh][c] * alpha[hh];
                for (int sl = 0; sl < nslots; ++sl) {
                    const float vv = vrow[sl];
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
    __syncthreads();
    merge_waves_and_store(a, w, lds, D);
}

template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
    combine_records<OutT>(a, blockIdx.x / a.num_kv_heads, blockIdx.x % a.num_kv_heads);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int q_dtype, int kv_dtype, hipStream_t s) {
    const long long grid = (long long)a.batch * a.chunks_per_seq;
    if (grid == 0) return hipSuccess;
    const size_t lds_merge = 4 * (32 + 16 * (size_t)a.head_dim) * sizeof(float);
    if (q_dtype == LSA_BF16 && kv_dtype == LSA_BF16) {
        if (a.head_dim == 128)
            hipLaunchKernelGGL(decode_bf16_kernel<128>, dim3((unsigned)grid), dim3(256), lds_merge, s, a);
        else
            hipLaunchKernelGGL(decode_bf16_kernel<64>, dim3((unsigned)grid), dim3(256), lds_merge, s, a);
    } else if (q_dtype == LSA_F32 && kv_dtype == LSA_F32) {
        const size_t lds = lds_merge + (16 * (size_t)a.head_dim + 4 * 16 * 64) * sizeof(float);
        if (a.head_dim == 128)
            hipLaunchKernelGGL(decode_f32_kernel<128>, dim3((unsigned)grid), dim3(256), lds, s, a);
        else
            hipLaunchKernelGGL(decode_f32_kernel<64>, dim3((unsigned)grid), dim3(256), lds, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


hipError_t launch_combine(const DecodeArgs &a, int q_dtype, hipStream_t s) {
    const long long grid = (long long)a.batch * a.num_kv_heads;
    if (grid == 0) return hipSuccess;
    if (q_dtype == LSA_BF16) hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace lsa
