// KV write through slot_mapping and the copy-on-write block copy.
//
// Write: "从零开始写Qwen3（六）PagedAttention", 自己来实现 -- token n's K and V rows
// (kvDim = Hkv*d values each) go to row slot_mapping[n] of the flat [num_blocks*B,
// kvDim] view of each pool; a negative slot means "do not write".
// Copy: "Paged attention 与 online softmax" §11.3 -- a shared block is copied to a new
// block before it is written.
//
// Both are pure data movement, bound by HBM bandwidth: one wave moves one row (or one
// slice of a block) with 16-byte loads and stores so that each wave instruction covers
// 1 KiB of consecutive bytes.

#include "common.h"

namespace pa {

constexpr int kWriteWaves = 4;  // tokens per workgroup

__global__ __launch_bounds__(kWriteWaves * kWave) void write_kv_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ slots, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int32_t n, int32_t row_vecs, int64_t capacity) {
    const int lane = threadIdx.x % kWave;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kWriteWaves + threadIdx.x / kWave;
    if (t >= n) return;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= capacity) return;  // skipped token (or out of range)
    const uint4* ks = k_new + t * row_vecs;
    const uint4* vs = v_new + t * row_vecs;
    uint4* kd = k_cache + slot * row_vecs;
    uint4* vd = v_cache + slot * row_vecs;
    for (int i = lane; i < row_vecs; i += kWave) {
        const uint4 a = ks[i];
        const uint4 b = vs[i];
        kd[i] = a;
        vd[i] = b;
    }
}

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int64_t block_vecs,
    int32_t num_blocks) {
    const int pair = blockIdx.y;
    const int32_t s = src[pair];
    const int32_t d = dst[pair];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
    const uint4* ks = k_cache + s * block_vecs;
    const uint4* vs = v_cache + s * block_vecs;
    uint4* kd = k_cache + d * block_vecs;
    uint4* vd = v_cache + d * block_vecs;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x; i < block_vecs;
         i += static_cast<int64_t>(gridDim.x) * kCopyThreads) {
        const uint4 a = ks[i];
        const uint4 b = vs[i];
        kd[i] = a;
        vd[i] = b;
    }
}

}  // namespace pa

extern "C" int pa_write_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, int32_t num_tokens, void* stream) {
    using namespace pa;
    int st = check_pool(pool);
    if (st != PA_OK) return st;
    if (num_tokens < 0) return PA_ERR_INVALID_ARG;
    if (num_tokens == 0) return PA_OK;
    if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr) return PA_ERR_INVALID_ARG;
    const int64_t row_bytes =
        static_cast<int64_t>(pool->num_kv_heads) * pool->head_dim * elem_bytes(pool->dtype);
    if (row_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
    const int64_t capacity = static_cast<int64_t>(pool->num_blocks) * pool->block_size;
    const dim3 grid((num_tokens + kWriteWaves - 1) / kWriteWaves);
    hipLaunchKernelGGL(write_kv_kernel, grid, dim3(kWriteWaves * kWave), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(k_new),
                       static_cast<const uint4*>(v_new), slot_mapping,
                       static_cast<uint4*>(pool->k_cache), static_cast<uint4*>(pool->v_cache),
                       num_tokens, static_cast<int32_t>(row_bytes / 16), capacity);
    return launch_status();
}

extern "C" int pa_copy_blocks(const pa_kv_pool* pool, const int32_t* src, const int32_t* dst,
                              int32_t num_pairs, void* stream) {
    using namespace pa;
    int st = check_pool(pool);
    if (st != PA_OK) return st;
    if (num_pairs < 0) return PA_ERR_INVALID_ARG;
    if (num_pairs == 0) return PA_OK;
    if (src == nullptr || dst == nullptr) return PA_ERR_INVALID_ARG;
    if (num_pairs > 65535) return PA_ERR_UNSUPPORTED;  // grid.y limit
    const int64_t block_bytes = static_cast<int64_t>(pool->block_size) * pool->num_kv_heads *
                                pool->head_dim * elem_bytes(pool->dtype);
    if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
    const int64_t vecs = block_bytes / 16;
    const int chunks = static_cast<int>((vecs + kCopyThreads * 4 - 1) / (kCopyThreads * 4));
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(chunks, num_pairs), dim3(kCopyThreads), 0,
                       static_cast<hipStream_t>(stream), src, dst,
                       static_cast<uint4*>(pool->k_cache), static_cast<uint4*>(pool->v_cache),
                       vecs, pool->num_blocks);
    return launch_status();
}
