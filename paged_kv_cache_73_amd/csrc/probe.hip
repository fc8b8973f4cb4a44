// Measurement helper: the attainable HBM read bandwidth of this GPU, for comparison with
// the attention kernels.  Every lane streams 16-byte pieces of a large buffer with
// non-temporal loads (the same load form as the decode pages) and folds them into a
// value that is stored only if it matches an impossible pattern, so nothing but the
// reads reaches memory.

#include "common.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n,
                                                          uint32_t* __restrict__ sink) {
    // Each workgroup reads its own contiguous stretch of the buffer (the last one also the
    // remainder): measured 7.0 TB/s on MI355X, against 6.2 TB/s for a grid-stride sweep of
    // the same buffer by the same grid.
    const int64_t per = n / gridDim.x;
    const int64_t b = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t e = blockIdx.x + 1 == gridDim.x ? n : b + per;
    uint32_t acc = 0;
#pragma unroll 8
    for (int64_t i = b + threadIdx.x; i < e; i += 256) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace pa

extern "C" int pa_probe_stream_read(const void* buf, size_t bytes, void* sink, int32_t grid,
                                    void* stream) {
    using namespace pa;
    if (buf == nullptr || sink == nullptr || grid <= 0 || bytes % 16 != 0) return PA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(buf), static_cast<int64_t>(bytes / 16),
                       static_cast<uint32_t*>(sink));
    return launch_status();
}
