// Paged decode for GQA group sizes 3, 5, 6 and 7 (query heads per KV head, as in models
// with 28 query heads over 4 KV heads) and 16 and 32 (a group spread over two or four
// waves of eight heads each).  The same kernel as for groups of 1, 2, 4 and 8
// (decode_kernel.h), instantiated here for head_dim 64 and 128 and block sizes 8, 16 and
// 32, plus one-row blocks for packed keys on the token path.  Other shapes with these
// group sizes return PA_ERR_UNSUPPORTED.

#include "decode_kernel.h"

namespace pa {

int decode_odd_groups(int G, const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                      int32_t num_heads, const int32_t* table, int32_t max_blocks,
                      const int32_t* seqlens, const void* k_new, const void* v_new,
                      int32_t max_parts, int32_t part_tokens, float scale, float* o_part,
                      float* ml_part, hipStream_t stream, const TokenMap& tm, int passes) {
    if (G != 3 && G != 5 && G != 6 && G != 7 && G != 16 && G != 32) return PA_ERR_UNSUPPORTED;
    const int D = pool->head_dim, BS = pool->block_size;
#define PA_DECODE_ODD(TT, DD, BB)                                                            \
    if (D == DD && BS == BB)                                                                 \
        return dispatch_group_odd<TT, DD, BB>(G, pool, out, q, batch, num_heads, table,      \
                                              max_blocks, seqlens, k_new, v_new, max_parts,  \
                                              part_tokens, scale, o_part, ml_part, stream, tm, \
                                              passes);
#define PA_DECODE_ODD_SHAPES(TT) \
    PA_DECODE_ODD(TT, 64, 16)    \
    PA_DECODE_ODD(TT, 64, 32)    \
    PA_DECODE_ODD(TT, 128, 16)   \
    PA_DECODE_ODD(TT, 128, 32)   \
    PA_DECODE_ODD(TT, 64, 8)     \
    PA_DECODE_ODD(TT, 128, 8)    \
    PA_DECODE_ODD(TT, 64, 1)     \
    PA_DECODE_ODD(TT, 128, 1)
    if (pool->dtype == PA_BF16) {
        PA_DECODE_ODD_SHAPES(bf16_t)
    } else {
        PA_DECODE_ODD_SHAPES(float)
    }
#undef PA_DECODE_ODD_SHAPES
#undef PA_DECODE_ODD
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa
