// Paged decode attention: host side of the two-pass split-K decode (partition choice,
// shape and group dispatch, argument checks, workspace) and the entry points of
// include/pa.h that use it.  The kernels and what they compute are in decode_kernel.h.

#include "decode_kernel.h"

namespace pa {

// Automatic split-K partition length.  A partition is one workgroup's share of a
// sequence; the aim is about kTargetWorkgroups workgroups in total (seven per CU of the
// 256 on an MI355X: enough to keep every CU fed, few enough that each streams a long
// run of pages and the merge stays small), assuming contexts average 60 % of the
// maximum, and no shorter than max_seqlen_k / kMaxAutoParts (to 64 tokens) so that the
// longest sequences are not cut into very many partitions -- unless so few sequences and
// KV-head groups that this would leave fewer than kMinWorkgroups workgroups (a single
// long sequence gets up to 256 partitions, none below 256 tokens).  Rounded to 64
// tokens and kept within [128, 4096].
constexpr int64_t kTargetWorkgroups = 7 * 256;
constexpr int64_t kMaxAutoParts = 64;
constexpr int64_t kMinWorkgroups = 1024;

// Keys per kernel step: a page, or for pages smaller than one 16-byte load per lane
// (block size 2 or 4) the rows one load covers (bf16's count, a multiple of fp32's).
inline int32_t step_keys(int32_t block_size, int32_t head_dim) {
    return std::max(block_size, 1024 / std::max(head_dim * 2, 1));
}

inline int32_t round_up(int32_t x, int32_t m) { return (x + m - 1) / m * m; }

inline int32_t pick_partition(int32_t partition_tokens, int32_t block_size, int32_t head_dim,
                              int32_t batch, int32_t num_kv_heads, int32_t max_seqlen_k) {
    const int32_t granule = step_keys(block_size, head_dim);
    if (partition_tokens > 0) return round_up(partition_tokens, granule);
    int per_wg = PA_DECODE_HPW;
    while (num_kv_heads % per_wg != 0) per_wg >>= 1;
    const int64_t groups = num_kv_heads / per_wg;
    const int64_t est_keys = static_cast<int64_t>(batch) * max_seqlen_k * 6 / 10;
    int64_t p = (est_keys * groups / kTargetWorkgroups + 63) / 64 * 64;
    // a bounded number of partitions per sequence: the merge reads each one's state
    const int64_t few = std::min<int64_t>(kMinWorkgroups / std::max<int64_t>(1, batch * groups),
                                          max_seqlen_k / 256);
    const int64_t max_auto_parts = std::max<int64_t>(kMaxAutoParts, few);
    p = std::max<int64_t>(p, (static_cast<int64_t>(max_seqlen_k) / max_auto_parts + 32) / 64 * 64);
    p = std::max<int64_t>(128, std::min<int64_t>(4096, p));
    return round_up(static_cast<int32_t>(p), granule);
}

// group sizes other than 1, 2, 4 and 8 (decode_groups.hip)
int decode_odd_groups(int G, const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                      int32_t num_heads, const int32_t* table, int32_t max_blocks,
                      const int32_t* seqlens, const void* k_new, const void* v_new,
                      int32_t max_parts, int32_t part_tokens, float scale, float* o_part,
                      float* ml_part, hipStream_t stream, const TokenMap& tm, int passes);


template <typename T>
int dispatch_shape(int G, const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                   int32_t num_heads, const int32_t* table, int32_t max_blocks,
                   const int32_t* seqlens, const void* k_new, const void* v_new, int32_t max_parts,
                   int32_t part_tokens, float scale, float* o_part, float* ml_part,
                   hipStream_t stream, const TokenMap& tm, int passes) {
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return decode_odd_groups(G, pool, out, q, batch, num_heads, table, max_blocks, seqlens,
                                 k_new, v_new, max_parts, part_tokens, scale, o_part, ml_part,
                                 stream, tm, passes);
    const int D = pool->head_dim, BS = pool->block_size;
#define PA_DECODE_SHAPE(DD, BB)                                                             \
    if (D == DD && BS == BB)                                                                \
        return dispatch_group_pow2<T, DD, BB>(G, pool, out, q, batch, num_heads, table, max_blocks, \
                                         seqlens, k_new, v_new, max_parts, part_tokens,       \
                                         scale, o_part, ml_part, stream, tm, passes);
    PA_DECODE_SHAPE(64, 16)
    PA_DECODE_SHAPE(64, 32)
    PA_DECODE_SHAPE(128, 16)
    PA_DECODE_SHAPE(128, 32)
    PA_DECODE_SHAPE(64, 8)
    PA_DECODE_SHAPE(128, 8)
    PA_DECODE_SHAPE(64, 4)
    PA_DECODE_SHAPE(128, 4)
    PA_DECODE_SHAPE(64, 2)
    PA_DECODE_SHAPE(128, 2)
    // head_dim 256: pages of up to 16 rows in bf16 and 8 in fp32 (larger pages hold too
    // many registers in the ping-pong buffers and spill)
    if constexpr (std::is_same<T, bf16_t>::value) {
        PA_DECODE_SHAPE(256, 16)
    }
    // one row per block: packed contiguous keys on the token path (and pools of B = 1)
    PA_DECODE_SHAPE(64, 1)
    PA_DECODE_SHAPE(128, 1)
    PA_DECODE_SHAPE(256, 1)
    PA_DECODE_SHAPE(256, 8)
    PA_DECODE_SHAPE(256, 4)
    PA_DECODE_SHAPE(256, 2)
#undef PA_DECODE_SHAPE
    return PA_ERR_UNSUPPORTED;
}

// large GQA groups in bf16 run on the matrix-core kernel of prefill.hip
bool decode_mc_shape(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size);
bool decode_on_matrix_cores(const pa_kv_pool* pool, int32_t num_heads);
size_t decode_mc_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seqlen_k, int32_t partition_tokens);
int decode_mc(const pa_kv_pool* pool, void* out, const void* q, const void* k_new,
              const void* v_new, int32_t batch, int32_t num_heads, const int32_t* table,
              int32_t max_blocks, const int32_t* seqlens, int32_t max_seqlen_k, float scale,
              int32_t partition_tokens, void* workspace, size_t workspace_size, hipStream_t s,
              int passes);

inline size_t workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim,
                              int32_t max_parts) {
    if (max_parts <= 1) return 0;
    return static_cast<size_t>(batch) * num_heads * max_parts * (head_dim + 2) * sizeof(float);
}

inline int32_t num_parts(int32_t max_seqlen_k, int32_t part_tokens) {
    return max_seqlen_k <= 0 ? 1 : (max_seqlen_k + part_tokens - 1) / part_tokens;
}

}  // namespace pa

extern "C" size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_seqlen_k, int32_t partition_tokens,
                                            int32_t block_size) {
    using namespace pa;
    if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
        return 0;
    const int32_t p = pick_partition(partition_tokens, block_size, head_dim, batch, num_kv_heads,
                                     max_seqlen_k);
    const size_t valu = workspace_bytes(batch, num_heads, head_dim, num_parts(max_seqlen_k, p));
    // the dtype is not known here: enough for either route
    if (!decode_mc_shape(num_heads, num_kv_heads, head_dim, block_size)) return valu;
    return std::max(valu, decode_mc_workspace_bytes(batch, num_heads, num_kv_heads, head_dim,
                                                    max_seqlen_k, partition_tokens));
}

namespace pa {

int decode_impl(const pa_kv_pool* pool, void* out, const void* q, const void* k_new,
                const void* v_new, int32_t batch, int32_t num_heads, const int32_t* block_table,
                int32_t max_blocks_per_seq, const int32_t* seqlens_k, int32_t max_seqlen_k,
                float softmax_scale, int32_t partition_tokens, void* workspace,
                size_t workspace_size, void* stream, int passes) {
    int st = check_pool(pool);
    if (st != PA_OK) return st;
    if (batch < 0 || num_heads <= 0 || max_blocks_per_seq < 0 || max_seqlen_k < 0 ||
        partition_tokens < 0)
        return PA_ERR_INVALID_ARG;
    if (batch == 0) return PA_OK;
    if (out == nullptr || seqlens_k == nullptr ||
        ((passes & kPass1) && (q == nullptr || (max_blocks_per_seq > 0 && block_table == nullptr))))
        return PA_ERR_INVALID_ARG;
    if (num_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (pool->num_kv_heads > 64) return PA_ERR_UNSUPPORTED;
    if (partition_tokens % pool->block_size != 0) return PA_ERR_INVALID_ARG;
    if (batch > 65535) return PA_ERR_UNSUPPORTED;
    {   // block sizes of the public calls (one-row blocks serve packed keys internally)
        const int32_t bs = pool->block_size;
        if (bs != 2 && bs != 4 && bs != 8 && bs != 16 && bs != 32) return PA_ERR_UNSUPPORTED;
    }
    if (decode_on_matrix_cores(pool, num_heads))
        return decode_mc(pool, out, q, k_new, v_new, batch, num_heads, block_table,
                         max_blocks_per_seq, seqlens_k, max_seqlen_k, softmax_scale,
                         partition_tokens, workspace, workspace_size,
                         static_cast<hipStream_t>(stream), passes);
    const int32_t part_tokens = pick_partition(partition_tokens, pool->block_size, pool->head_dim,
                                               batch, pool->num_kv_heads, max_seqlen_k);
    if (part_tokens % pool->block_size != 0) return PA_ERR_INVALID_ARG;
    // keys beyond the table width are never read, so the width also bounds the grid
    const int64_t cap = static_cast<int64_t>(max_blocks_per_seq) * pool->block_size;
    const int32_t eff_max = static_cast<int32_t>(std::min<int64_t>(max_seqlen_k, cap));
    const int32_t max_parts = num_parts(eff_max, part_tokens);
    if (max_parts > 65535) return PA_ERR_UNSUPPORTED;  // grid.y limit
    const size_t need = workspace_bytes(batch, num_heads, pool->head_dim, max_parts);
    if (need > 0 && (workspace == nullptr || workspace_size < need)) return PA_ERR_WORKSPACE;
    float* o_part = static_cast<float*>(workspace);
    float* ml_part = need ? o_part + static_cast<size_t>(batch) * num_heads * max_parts * pool->head_dim
                          : nullptr;
    const int G = num_heads / pool->num_kv_heads;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (pool->dtype == PA_BF16)
        return dispatch_shape<bf16_t>(G, pool, out, q, batch, num_heads, block_table,
                                      max_blocks_per_seq, seqlens_k, k_new, v_new, max_parts,
                                      part_tokens, softmax_scale, o_part, ml_part, s, TokenMap{},
                                      passes);
    return dispatch_shape<float>(G, pool, out, q, batch, num_heads, block_table,
                                 max_blocks_per_seq, seqlens_k, k_new, v_new, max_parts,
                                 part_tokens, softmax_scale, o_part, ml_part, s, TokenMap{}, passes);
}

// The varlen prefill run one packed query token at a time by the decode kernel, each
// token over its request's keys in a single partition (no workspace).  No matrix cores:
// the path for pools the MFMA prefill does not take (fp32).  Arguments as for
// pa_prefill_varlen, already checked by it.
int prefill_by_token(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                     int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                     int32_t max_seqlen_q, const int32_t* block_table, int32_t max_blocks,
                     float scale, int32_t causal, hipStream_t s, int32_t contiguous) {
    if (pool->num_kv_heads > 64) return PA_ERR_UNSUPPORTED;
    const int32_t part_tokens =  // one partition
        round_up(std::max(max_blocks, 1) * pool->block_size, step_keys(pool->block_size, pool->head_dim));
    const int G = num_heads / pool->num_kv_heads;
    const int64_t bound = static_cast<int64_t>(batch) * max_seqlen_q;  // tokens, at most
    for (int64_t first = 0; first < bound; first += 65535) {
        const int32_t n = static_cast<int32_t>(std::min<int64_t>(65535, bound - first));
        TokenMap tm;
        tm.cu_q = cu_q;
        tm.cu_k = cu_k;
        tm.n_req = batch;
        tm.causal = causal != 0;
        tm.offset = static_cast<int32_t>(first);
        tm.max_q = max_seqlen_q;
        tm.contiguous = contiguous;
        const int st = pool->dtype == PA_BF16
            ? dispatch_shape<bf16_t>(G, pool, out, q, n, num_heads, block_table, max_blocks,
                                     nullptr, nullptr, nullptr, 1, part_tokens, scale, nullptr,
                                     nullptr, s, tm, kPass1 | kPass2)
            : dispatch_shape<float>(G, pool, out, q, n, num_heads, block_table, max_blocks,
                                    nullptr, nullptr, nullptr, 1, part_tokens, scale, nullptr,
                                    nullptr, s, tm, kPass1 | kPass2);
        if (st != PA_OK) return st;
    }
    return PA_OK;
}

}  // namespace pa

extern "C" int pa_decode(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                         int32_t num_heads, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* seqlens_k,
                         int32_t max_seqlen_k, float softmax_scale, int32_t partition_tokens,
                         void* workspace, size_t workspace_size, void* stream) {
    return pa::decode_impl(pool, out, q, nullptr, nullptr, batch, num_heads, block_table,
                           max_blocks_per_seq, seqlens_k, max_seqlen_k, softmax_scale,
                           partition_tokens, workspace, workspace_size, stream,
                           pa::kPass1 | pa::kPass2);
}

extern "C" int pa_decode_partials(const pa_kv_pool* pool, void* out, const void* q,
                                  const void* k_new, const void* v_new, int32_t batch,
                                  int32_t num_heads, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, const int32_t* seqlens_k,
                                  int32_t max_seqlen_k, float softmax_scale,
                                  int32_t partition_tokens, void* workspace,
                                  size_t workspace_size, void* stream) {
    if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_INVALID_ARG;
    return pa::decode_impl(pool, out, q, k_new, v_new, batch, num_heads, block_table,
                           max_blocks_per_seq, seqlens_k, max_seqlen_k, softmax_scale,
                           partition_tokens, workspace, workspace_size, stream, pa::kPass1);
}

extern "C" int pa_decode_merge(const pa_kv_pool* pool, void* out, int32_t batch, int32_t num_heads,
                               int32_t max_blocks_per_seq, const int32_t* seqlens_k,
                               int32_t max_seqlen_k, int32_t partition_tokens, void* workspace,
                               size_t workspace_size, void* stream) {
    return pa::decode_impl(pool, out, nullptr, nullptr, nullptr, batch, num_heads, nullptr,
                           max_blocks_per_seq, seqlens_k, max_seqlen_k, 1.f, partition_tokens,
                           workspace, workspace_size, stream, pa::kPass2);
}

extern "C" int pa_decode_append(const pa_kv_pool* pool, void* out, const void* q,
                                const void* k_new, const void* v_new, int32_t batch,
                                int32_t num_heads, const int32_t* block_table,
                                int32_t max_blocks_per_seq, const int32_t* seqlens_k,
                                int32_t max_seqlen_k, float softmax_scale,
                                int32_t partition_tokens, void* workspace, size_t workspace_size,
                                void* stream) {
    if (batch > 0 && (k_new == nullptr || v_new == nullptr)) return PA_ERR_INVALID_ARG;
    return pa::decode_impl(pool, out, q, k_new, v_new, batch, num_heads, block_table,
                           max_blocks_per_seq, seqlens_k, max_seqlen_k, softmax_scale,
                           partition_tokens, workspace, workspace_size, stream,
                           pa::kPass1 | pa::kPass2);
}
