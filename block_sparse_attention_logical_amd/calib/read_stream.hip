// Calibration kernel (not part of liblsa): a plain streaming read of one
// contiguous buffer, to measure what HBM sustains for a read of a given size
// on this part, ramp-up and tail included.  Each workgroup reads a contiguous
// slab with 16-byte non-temporal loads, eight in flight per thread, and folds
// the words into one value that is stored only if it equals a sentinel, so
// the loads are kept and the kernel writes (practically) nothing.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4 *__restrict__ src, size_t n16,
                                                               size_t per_wg, uint32_t *__restrict__ out) {
    const size_t base = (size_t)blockIdx.x * per_wg;
    const size_t end = base + per_wg < n16 ? base + per_wg : n16;
    uint32_t acc = 0;
    for (size_t i = base + threadIdx.x; i < end; i += (size_t)kThreads * kInFlight) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const size_t j = i + (size_t)u * kThreads;
            v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) from `src` with `grid` workgroups on
// `stream`; out: at least grid uint32 of device memory.  Returns a hipError_t.
extern "C" int calib_read_stream(const void *src, size_t bytes, int grid, void *out, void *stream) {
    if (grid <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
    const size_t n16 = bytes / 16;
    const size_t per_wg = (n16 + grid - 1) / grid;
    hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u32x4 *>(src), n16, per_wg, static_cast<uint32_t *>(out));
    return (int)hipGetLastError();
}
