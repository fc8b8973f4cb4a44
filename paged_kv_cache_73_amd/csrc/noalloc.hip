// pa_decode_noalloc: pa_decode with its split-K scratch (the partial states of the
// sequences cut into partitions, and on the matrix-core route the device-built sequence
// offsets) in a static device array of the library instead of a caller's workspace, for
// callers that cannot allocate device memory.  Everything else is pa_decode's path.

#include <atomic>

#include "common.h"

namespace pa {
namespace {

constexpr size_t kScratchBytes = PA_DECODE_SCRATCH_BYTES;

// One per GPU the library runs on, alive until the process ends.  Its contents need no
// initialisation: pa_decode writes every partial state it later reads.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The array's device address on each GPU, looked up on the first call made with that GPU
// current.  (In host code the name scratch stands for a host-side shadow, not a device
// address: kernels get this pointer.)
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_on[kMaxDevices];

int scratch_ptr(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    void* p = scratch_on[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return PA_ERR_HIP;
        scratch_on[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" int pa_decode_noalloc(const pa_kv_pool* pool, void* out, const void* q,
                                 int32_t batch, int32_t num_heads, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* seqlens_k,
                                 int32_t max_seqlen_k, float softmax_scale,
                                 int32_t partition_tokens, void* stream) {
    if (pool == nullptr) return PA_ERR_INVALID_ARG;
    // the scratch a pa_decode of these arguments needs (0 when nothing is split); more
    // than the static array holds is refused before anything runs
    const size_t need = pa_decode_workspace_bytes(batch, num_heads, pool->num_kv_heads,
                                                  pool->head_dim, max_seqlen_k,
                                                  partition_tokens, pool->block_size);
    if (need > pa::kScratchBytes) return PA_ERR_WORKSPACE;
    void* ws = nullptr;
    const int st = pa::scratch_ptr(&ws);
    if (st != PA_OK) return st;
    return pa_decode(pool, out, q, batch, num_heads, block_table, max_blocks_per_seq, seqlens_k,
                     max_seqlen_k, softmax_scale, partition_tokens, ws, pa::kScratchBytes,
                     stream);
}
