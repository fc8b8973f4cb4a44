// Varlen paged prefill (MFMA); filled in by the prefill kernel.
#include "common.h"

extern "C" int pa_prefill_varlen(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                                 int32_t num_heads, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, float softmax_scale, int32_t causal,
                                 void* stream) {
    (void)pool; (void)out; (void)q; (void)batch; (void)num_heads; (void)cu_seqlens_q;
    (void)cu_seqlens_k; (void)max_seqlen_q; (void)max_seqlen_k; (void)block_table;
    (void)max_blocks_per_seq; (void)softmax_scale; (void)causal; (void)stream;
    return PA_ERR_UNSUPPORTED;
}
