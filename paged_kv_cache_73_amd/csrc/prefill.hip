// Varlen (packed) paged prefill on the matrix cores: host launch code, the merge of
// key-split ranges, and decode with large GQA groups on the same kernel.  The kernel and
// its design are in prefill_kernel.h.

#include <algorithm>
#include <atomic>

#include "common.h"
#include "prefill_launch.h"

namespace pa {

// The varlen prefill run token by token on the decode kernel (decode.hip): the path
// for fp32 pools.
int prefill_by_token(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                     int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                     int32_t max_seqlen_q, const int32_t* block_table, int32_t max_blocks,
                     float scale, int32_t causal, hipStream_t s, int32_t contiguous);


// Key splitting (pa_prefill_varlen_splitk).  A job walks all its key tiles in one
// workgroup, so when a batch has fewer jobs than the GPU has workgroup slots (two per CU),
// the longest jobs alone set the time while most slots idle.  Such batches have their
// jobs cut into key ranges, and a merge pass folds the ranges.  With the lengths on the
// host and at most half as many jobs as slots (a chunk of one long prompt, a few
// requests), ranges of about (all jobs' tiles) / slots tiles, at least
// kMinSplitTilesExact, leave about one range per slot.  Otherwise (or with only the
// bounds max_seqlen_q and max_seqlen_k) ranges of at least kMinSplitTiles tiles aim at
// kSplitTargetUnits ranges for jobs of the longest length: mixed lengths then split
// only their longest jobs, since every extra range adds its partial state (128 rows x
// (d + 2) floats written, then read by the merge) and a workgroup's fixed costs.  The
// plan depends only on the host arguments, so the workspace query and the call agree.
constexpr int64_t kSplitBelowJobs = 1024;  // a bound on the jobs from which none is split
constexpr int64_t kSplitTargetUnits = 1024;
constexpr int64_t kMinSplitTiles = 1024 / kPrefillKeys;      // tiles of a range: 1024 keys
constexpr int64_t kMinSplitTilesExact = 512 / kPrefillKeys;  // 512 keys

inline SplitPlan plan_split(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, bool causal,
                            const int32_t* host_cu_q, const int32_t* host_cu_k) {
    SplitPlan p{1, 0, 0};
    if (batch <= 0 || num_kv_heads <= 0 || num_heads < num_kv_heads) return p;
    const int64_t tok = std::max(kPrefillRows / (num_heads / num_kv_heads), 1);
    const int64_t n_qtiles = (max_seqlen_q + tok - 1) / tok;
    const int64_t dense = static_cast<int64_t>(batch) * num_kv_heads * n_qtiles;
    if (dense == 0) return p;
    int64_t st = 0, longest = 0;
    if (host_cu_q != nullptr && host_cu_k != nullptr) {
        // every job's key tiles, as the kernel counts them (without the table-width cap)
        int64_t jobs = 0, tiles = 0;
        for (int32_t i = 0; i < batch; ++i) {
            const int64_t q_len = host_cu_q[i + 1] - host_cu_q[i];
            const int64_t k_len = host_cu_k[i + 1] - host_cu_k[i];
            for (int64_t t0 = 0; t0 < std::min<int64_t>(q_len, max_seqlen_q); t0 += tok) {
                const int64_t last = std::min(t0 + tok, q_len) - 1;
                const int64_t kv_end = causal ? std::min(k_len, k_len - q_len + last + 1) : k_len;
                const int64_t t = kv_end > 0 ? (kv_end + kPrefillKeys - 1) / kPrefillKeys : 0;
                jobs += num_kv_heads;
                tiles += t * num_kv_heads;
                longest = std::max(longest, t);
            }
        }
        if (jobs == 0 || jobs >= prefill_slots()) return p;
        if (2 * jobs <= prefill_slots())
            st = std::max<int64_t>(kMinSplitTilesExact, (tiles + prefill_slots() - 1) / prefill_slots());
    }
    if (st == 0) {
        longest = std::max(longest, (static_cast<int64_t>(max_seqlen_k) + kPrefillKeys - 1) / kPrefillKeys);
        if (dense >= kSplitBelowJobs) return p;
        st = std::max<int64_t>(kMinSplitTiles, (longest * dense + kSplitTargetUnits - 1) / kSplitTargetUnits);
    }
    if (longest <= st) return p;
    p.n_split = static_cast<int32_t>((longest + st - 1) / st);
    p.split_tiles = static_cast<int32_t>(st);
    p.units = dense * p.n_split;
    return p;
}

inline size_t split_workspace_bytes(const SplitPlan& p, int32_t head_dim) {
    if (p.n_split <= 1) return 0;
    return static_cast<size_t>(p.units) * kPrefillRows * (static_cast<size_t>(head_dim) * 4 + 8);
}



int prefill_impl(const KvSource& kv, int32_t head_dim, void* out, const void* q, int32_t batch,
                 int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                 int32_t max_seqlen_q, float scale, int32_t causal, hipStream_t s,
                 const SplitPlan& sp = SplitPlan{1, 0, 0}, void* workspace = nullptr,
                 int passes = kPass1 | kPass2) {
    if (num_heads % kv.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || scale == INFINITY) return PA_ERR_INVALID_ARG;
    const int G = num_heads / kv.num_kv_heads;
    const int32_t c = causal != 0;
    if (head_dim == 128) {
        const bool pow2 = G == 1 || G == 2 || G == 4 || G == 8;
        return (pow2 ? prefill_dispatch_k128 : prefill_dispatch_k128_odd)(
            G, kv, out, q, batch, num_heads, cu_q, cu_k, max_seqlen_q, scale, c, s, sp,
            workspace, passes);
    }
    if (head_dim == 64)
        return prefill_dispatch_k64(G, kv, out, q, batch, num_heads, cu_q, cu_k, max_seqlen_q,
                                    scale, c, s, sp, workspace, passes);
    return PA_ERR_UNSUPPORTED;
}

// ---------------------------------------------------------------------------------------
// Decode with large GQA groups on the matrix cores.  The decode kernel (decode_kernel.h)
// computes each lane's dot products on the vector unit, G query heads at a time; from
// five query heads per KV head on, that vector work, not HBM, sets its pace (64 query /
// 8 KV heads: 2.4 TB/s).  A decode step is also a varlen prefill with one query token
// per sequence: the G heads of a KV head are G rows of one job of this file's kernel,
// whose products run on the matrix cores, with a key-split plan in place of the decode
// partitions.  pa_decode, its two passes and pa_decode_append take this route for such
// shapes; the workspace holds cu_seqlens built from seqlens, then the split states.
// ---------------------------------------------------------------------------------------

constexpr int kDecodeMcMinGroup = 5;

// the shapes (dtype aside: bf16 only) that take this route
bool decode_mc_shape(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size) {
    if (num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return false;
    const int G = num_heads / num_kv_heads;
    const bool group = (G >= kDecodeMcMinGroup && G <= 8) || G == 16 || G == 32;
    return group && (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32);
}

bool decode_on_matrix_cores(const pa_kv_pool* pool, int32_t num_heads) {
    return pool->dtype == PA_BF16 &&
           decode_mc_shape(num_heads, pool->num_kv_heads, pool->head_dim, pool->block_size);
}

inline size_t decode_mc_header(int32_t batch) {
    return (2 * (static_cast<size_t>(batch) + 1) * sizeof(int32_t) + 255) / 256 * 256;
}

// Key ranges: of partition_tokens keys (rounded up to whole key tiles) when given.
// Else ranges long enough for about kDecodeTargetUnits (job, range) units over the
// longest sequence, of at least kDecodeMinSplitTiles tiles, and of up to kDecodeSplitTiles
// while that still leaves kDecodeFewUnits units: a decode job has one query row per head,
// so a range's fixed costs weigh more than in a prefill.  (Measured on 64 query / 8 or 4
// KV heads: 4 sequences of 16K keys and 16 of 8K ran fastest in ranges of 12-16 tiles,
// 64 sequences of 4K in two ranges rather than four, 8 of 40K in 16 ranges of 40 tiles;
// 8 sequences of 4K with 40 / 8 heads in ranges of 8 tiles, 29 against 37 us at 16.)
constexpr int64_t kDecodeTargetUnits = 1024;
constexpr int64_t kDecodeFewUnits = 512;
constexpr int64_t kDecodeMinSplitTiles = 512 / kPrefillKeys;   // 512 keys
constexpr int64_t kDecodeSplitTiles = 2048 / kPrefillKeys;     // 2048 keys

inline SplitPlan decode_mc_plan(int32_t batch, int32_t num_kv_heads, int32_t max_seqlen_k,
                                int32_t partition_tokens) {
    SplitPlan p{1, 0, 0};
    const int64_t longest = (static_cast<int64_t>(max_seqlen_k) + kPrefillKeys - 1) / kPrefillKeys;
    const int64_t work = longest * batch * num_kv_heads;  // tiles of the longest jobs
    const int64_t st = partition_tokens > 0
        ? (static_cast<int64_t>(partition_tokens) + kPrefillKeys - 1) / kPrefillKeys
        : std::max({kDecodeMinSplitTiles, (work + kDecodeTargetUnits - 1) / kDecodeTargetUnits,
                    std::min(kDecodeSplitTiles, work / kDecodeFewUnits)});
    if (longest <= st) return p;
    p.n_split = static_cast<int32_t>((longest + st - 1) / st);
    p.split_tiles = static_cast<int32_t>(st);
    p.units = static_cast<int64_t>(batch) * num_kv_heads * p.n_split;
    return p;
}

size_t decode_mc_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seqlen_k, int32_t partition_tokens) {
    return decode_mc_header(batch) +
           split_workspace_bytes(decode_mc_plan(batch, num_kv_heads, max_seqlen_k, partition_tokens),
                                 head_dim);
}

// cu_q[i] = i; cu_k = running sum of max(seqlens, 0), kept modulo 2^32 (only
// differences of consecutive entries are read).  One wave: each lane sums a run of
// sequences, a shuffle scan gives the lanes' offsets.
__global__ __launch_bounds__(kWave) void decode_cu_kernel(const int32_t* __restrict__ seqlens,
                                                          int32_t batch, int32_t* __restrict__ cu_q,
                                                          int32_t* __restrict__ cu_k) {
    const int t = threadIdx.x;
    const int per = (batch + kWave - 1) / kWave;
    const int lo = min(t * per, batch), hi = min(lo + per, batch);
    uint32_t sum = 0;
    for (int i = lo; i < hi; ++i) sum += static_cast<uint32_t>(max(seqlens[i], 0));
    uint32_t incl = sum;  // inclusive scan over the lanes
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (t >= off) incl += v;
    }
    uint32_t run = incl - sum;
    for (int i = lo; i < hi; ++i) {
        cu_k[i] = static_cast<int32_t>(run);
        cu_q[i] = i;
        run += static_cast<uint32_t>(max(seqlens[i], 0));
    }
    if (t == kWave - 1) {
        cu_k[batch] = static_cast<int32_t>(incl);
        cu_q[batch] = batch;
    }
}

// pa_decode_append's write on this route: the new K/V row of sequence b goes to position
// seqlens[b] - 1 through its table row (skipped when that block is unassigned), as the
// decode kernel's fused append stores it.  One workgroup per sequence.
__global__ __launch_bounds__(kWave) void decode_append_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ table, int32_t max_blocks,
    int32_t block_size, int32_t num_blocks, int32_t row_vecs, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache) {
    const int b = blockIdx.x;
    const int64_t cap = static_cast<int64_t>(max_blocks) * block_size;
    const int64_t len = min(static_cast<int64_t>(max(seqlens[b], 0)), cap);
    if (len <= 0) return;
    const int64_t pos = len - 1;
    const int32_t id = table[static_cast<int64_t>(b) * max_blocks + pos / block_size];
    if (id < 0 || id >= num_blocks) return;
    const int64_t slot = static_cast<int64_t>(id) * block_size + pos % block_size;
    for (int i = threadIdx.x; i < row_vecs; i += kWave) {
        k_cache[slot * row_vecs + i] = k_new[static_cast<int64_t>(b) * row_vecs + i];
        v_cache[slot * row_vecs + i] = v_new[static_cast<int64_t>(b) * row_vecs + i];
    }
}

int decode_mc(const pa_kv_pool* pool, void* out, const void* q, const void* k_new,
              const void* v_new, int32_t batch, int32_t num_heads, const int32_t* table,
              int32_t max_blocks, const int32_t* seqlens, int32_t max_seqlen_k, float scale,
              int32_t partition_tokens, void* workspace, size_t workspace_size, hipStream_t s,
              int passes) {
    // checked before any launch, so that a refused call leaves the pool untouched
    if ((passes & kPass1) && (!(scale > 0.f) || scale == INFINITY)) return PA_ERR_INVALID_ARG;
    const SplitPlan sp = decode_mc_plan(batch, pool->num_kv_heads, max_seqlen_k, partition_tokens);
    const size_t need = decode_mc_header(batch) + split_workspace_bytes(sp, pool->head_dim);
    if (workspace == nullptr || workspace_size < need) return PA_ERR_WORKSPACE;
    int32_t* cu_q = static_cast<int32_t*>(workspace);
    int32_t* cu_k = cu_q + batch + 1;
    void* states = static_cast<char*>(workspace) + decode_mc_header(batch);
    if (passes & kPass1) {
        hipLaunchKernelGGL(decode_cu_kernel, dim3(1), dim3(kWave), 0, s, seqlens, batch, cu_q, cu_k);
        if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
        if (k_new != nullptr) {
            const int32_t row_vecs = pool->num_kv_heads * pool->head_dim * 2 / 16;
            hipLaunchKernelGGL(decode_append_kernel, dim3(batch), dim3(kWave), 0, s,
                               static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                               seqlens, table, max_blocks, pool->block_size, pool->num_blocks,
                               row_vecs, static_cast<uint4*>(pool->k_cache),
                               static_cast<uint4*>(pool->v_cache));
            if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
        }
    } else if (sp.n_split <= 1) {
        return PA_OK;  // the first pass finished every row
    }
    const KvSource kv{true, pool->k_cache, pool->v_cache, pool->num_kv_heads, pool->num_blocks,
                      pool->block_size, table, max_blocks};
    // one query token per sequence, all its keys visible (non-causal is the same here)
    return prefill_impl(kv, pool->head_dim, out, q, batch, num_heads, cu_q, cu_k, 1,
                        scale, 0, s, sp, states, passes);
}

}  // namespace pa

namespace pa {

// the paged pool's calls take the matrix cores for BF16 pools of head_dim <= 128 with
// blocks of 16 or 32 rows; the rest runs token by token
inline bool on_matrix_cores(int32_t dtype, int32_t block_size, int32_t head_dim) {
    return dtype == PA_BF16 && block_size >= 16 && head_dim <= 128;
}

int paged_prefill(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                  int32_t num_heads, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int32_t max_seqlen_q, int32_t max_seqlen_k, const int32_t* block_table,
                  int32_t max_blocks_per_seq, float softmax_scale, int32_t causal, void* stream,
                  bool may_split, const int32_t* host_cu_q, const int32_t* host_cu_k,
                  void* workspace, size_t workspace_bytes) {
    int st = check_pool(pool);
    if (st != PA_OK) return st;
    if (batch < 0 || num_heads <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0 ||
        max_blocks_per_seq < 0)
        return PA_ERR_INVALID_ARG;
    if (batch == 0 || max_seqlen_q == 0) return PA_OK;
    if (out == nullptr || q == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr ||
        (max_blocks_per_seq > 0 && block_table == nullptr))
        return PA_ERR_INVALID_ARG;
    const int32_t bs = pool->block_size;
    if (bs != 2 && bs != 4 && bs != 8 && bs != 16 && bs != 32) return PA_ERR_UNSUPPORTED;
    if (pool->dtype == PA_F32 || bs < 16 || pool->head_dim > 128) {  // not on the matrix cores
        if (num_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
        if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return PA_ERR_INVALID_ARG;
        return prefill_by_token(pool, out, q, batch, num_heads, cu_seqlens_q, cu_seqlens_k,
                                max_seqlen_q, block_table, max_blocks_per_seq, softmax_scale,
                                causal, static_cast<hipStream_t>(stream), 0);
    }
    if (pool->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    // without splitting the per-request lengths alone bound the key loop; the split plan
    // reads max_seqlen_k (ranges past it would not be walked: a caller error)
    SplitPlan sp{1, 0, 0};
    if (may_split) {
        sp = plan_split(batch, num_heads, pool->num_kv_heads, max_seqlen_q, max_seqlen_k,
                        causal != 0, host_cu_q, host_cu_k);
        const size_t need = split_workspace_bytes(sp, pool->head_dim);
        if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    }
    // a table of width 0 (possibly null) assigns no block: every row outputs zeros, and
    // the kernel reads no table entry because no request then has a key to load
    const KvSource kv{true, pool->k_cache, pool->v_cache, pool->num_kv_heads, pool->num_blocks,
                      pool->block_size, block_table, max_blocks_per_seq};
    return prefill_impl(kv, pool->head_dim, out, q, batch, num_heads, cu_seqlens_q, cu_seqlens_k,
                        max_seqlen_q, softmax_scale, causal, static_cast<hipStream_t>(stream), sp,
                        workspace);
}

}  // namespace pa

extern "C" int pa_prefill_varlen(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                                 int32_t num_heads, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, float softmax_scale, int32_t causal,
                                 void* stream) {
    return pa::paged_prefill(pool, out, q, batch, num_heads, cu_seqlens_q, cu_seqlens_k,
                             max_seqlen_q, max_seqlen_k, block_table, max_blocks_per_seq,
                             softmax_scale, causal, stream, false, nullptr, nullptr, nullptr, 0);
}

extern "C" size_t pa_prefill_workspace_bytes(int32_t dtype, int32_t batch, int32_t num_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_seqlen_q,
                                             int32_t max_seqlen_k, int32_t causal,
                                             const int32_t* host_cu_seqlens_q,
                                             const int32_t* host_cu_seqlens_k) {
    using namespace pa;
    if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seqlen_q <= 0 ||
        max_seqlen_k < 0 || num_heads % num_kv_heads != 0)
        return 0;
    if (!on_matrix_cores(dtype, block_size, head_dim)) return 0;
    return split_workspace_bytes(plan_split(batch, num_heads, num_kv_heads, max_seqlen_q,
                                            max_seqlen_k, causal != 0, host_cu_seqlens_q,
                                            host_cu_seqlens_k),
                                 head_dim);
}

extern "C" int pa_prefill_varlen_splitk(const pa_kv_pool* pool, void* out, const void* q,
                                        int32_t batch, int32_t num_heads,
                                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                        int32_t max_seqlen_q, int32_t max_seqlen_k,
                                        const int32_t* block_table, int32_t max_blocks_per_seq,
                                        float softmax_scale, int32_t causal,
                                        const int32_t* host_cu_seqlens_q,
                                        const int32_t* host_cu_seqlens_k, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    return pa::paged_prefill(pool, out, q, batch, num_heads, cu_seqlens_q, cu_seqlens_k,
                             max_seqlen_q, max_seqlen_k, block_table, max_blocks_per_seq,
                             softmax_scale, causal, stream, true, host_cu_seqlens_q,
                             host_cu_seqlens_k, workspace, workspace_bytes);
}

extern "C" int pa_prefill_varlen_contiguous(void* out, const void* q, const void* k,
                                            const void* v, int32_t dtype, int32_t batch,
                                            int32_t num_heads, int32_t num_kv_heads,
                                            int32_t head_dim, const int32_t* cu_seqlens_q,
                                            const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                                            int32_t max_seqlen_k, float softmax_scale,
                                            int32_t causal, void* stream) {
    using namespace pa;
    if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seqlen_q < 0 ||
        max_seqlen_k < 0)
        return PA_ERR_INVALID_ARG;
    if (dtype != PA_BF16 && dtype != PA_F32) return PA_ERR_INVALID_ARG;
    if (batch == 0 || max_seqlen_q == 0) return PA_OK;
    if (out == nullptr || q == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr ||
        (max_seqlen_k > 0 && (k == nullptr || v == nullptr)))
        return PA_ERR_INVALID_ARG;
    if (dtype != PA_BF16 || head_dim > 128) {
        // fp32, or head_dim 256: the token path, the packed rows seen as a pool of one-row
        // blocks in which key j of request i is block cu_k[i] + j (no table is read)
        if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
        if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return PA_ERR_INVALID_ARG;
        const pa_kv_pool rows{dtype, INT32_MAX, 1, num_kv_heads, head_dim, const_cast<void*>(k),
                              const_cast<void*>(v)};
        return prefill_by_token(&rows, out, q, batch, num_heads, cu_seqlens_q, cu_seqlens_k,
                                max_seqlen_q, nullptr, std::max(max_seqlen_k, 1), softmax_scale,
                                causal, static_cast<hipStream_t>(stream), 1);
    }
    const KvSource kv{false, k, v, num_kv_heads, 0, 0, nullptr, 0};
    return prefill_impl(kv, head_dim, out, q, batch, num_heads, cu_seqlens_q, cu_seqlens_k,
                        max_seqlen_q, softmax_scale, causal, static_cast<hipStream_t>(stream));
}
