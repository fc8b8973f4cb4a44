/*
 * pa.h -- C ABI of libpa, paged attention over a block-table-indexed KV cache for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [PA11]  "Paged attention 与 online softmax" (dilfish.github.io, chapter 11):
 *           §11.1 block table / address / pool size, §11.2 block-merge online
 *           softmax, §11.3 sharing, copy-on-write, reference counts.
 *   [NANO]  "结合nanovllm的FlashAttention和PagedAttention主要原理概述"
 *           (meredith2328.github.io): 题目2 online softmax, 题目3 FlashAttention tiles,
 *           题目4 on-demand blocks, 题目5 block table, 题目6 prefix reference counts.
 *   [QWEN]  "从零开始写Qwen3（六）PagedAttention" (mlqm.cn reprint): 分页自注意力的改进
 *           (address rule), packed 模式, fast-attn 库的使用 (varlen prefill and decode
 *           call signatures), 自己来实现 (slot_mapping write).
 *   [HFPA]  "Sayfalı dikkat" (Hugging Face transformers docs, Turkish): varlen path
 *           (Değişken uzunluklu yol) and decode path (Çözme yolu) with examples.
 *
 * Conventions shared by every call
 * --------------------------------
 * - KV pools: two caller-owned device buffers, K and V, each laid out
 *   [num_blocks][block_size][num_kv_heads][head_dim], row-major, head_dim fastest
 *   ([PA11] §11.1: the K vector of (phys, slot) starts at phys*B*kvDim + slot*kvDim,
 *   kvDim = num_kv_heads*head_dim).  Element type pa_dtype.
 * - A logical token p of sequence s lives in physical block table[s][p / B] at slot
 *   p % B ([PA11] §11.1, [NANO] 题目5); its flat slot index is table[s][p/B]*B + p%B
 *   ([QWEN] 分页自注意力的改进).
 * - Block tables: int32 [batch][max_blocks_per_seq] on the device, unassigned entries
 *   -1 ([HFPA] decode example).  Entries outside [0, num_blocks) within a sequence's
 *   length are a caller error; the kernels never dereference them: such blocks are
 *   treated as masked (their keys take no part), keeping every access in bounds.
 * - Query head h uses KV head h / (num_heads / num_kv_heads) (grouped-query attention).
 * - Every device call enqueues asynchronously on `stream` (a hipStream_t; NULL is the
 *   default stream), never synchronises, never allocates device memory and keeps no
 *   state between calls.  All pointers named "device" must be device memory that
 *   stays valid until the enqueued work completes.
 * - Every call returns a pa_status.  Scalar arguments are validated on the host
 *   before anything is launched; on error nothing is enqueued.  A failed launch
 *   returns PA_ERR_HIP.  The contents of device metadata (tables, lengths, slots)
 *   are not validated by the device calls (that would need a synchronisation);
 *   the pa_validate_* functions check host copies of them.
 * - Supported: dtype F32 or BF16, head_dim 64 or 128, block_size 2, 4, 8, 16 or 32,
 *   group size G = num_heads / num_kv_heads from 1 to 8, 16 or 32, num_kv_heads <= 64;
 *   head_dim 256 too for the decode calls and the paged prefill, with block_size up to 16
 *   (BF16) or 8 (F32).  Group sizes 3, 5, 6, 7, 16 and 32 need head_dim 64 or 128 and
 *   block_size 8, 16 or 32 wherever the decode kernel runs (decode calls, and the
 *   prefill's token path below).  Other shapes return PA_ERR_UNSUPPORTED.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1,   /* null pointer, negative size, inconsistent shapes  */
    PA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (dtype, head_dim, ...)  */
    PA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required        */
    PA_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed        */
    PA_ERR_OUT_OF_BLOCKS = -5, /* block manager: not enough free blocks             */
    PA_ERR_REFCOUNT = -6,      /* block manager: reference count would go below 0   */
    PA_ERR_METADATA = -7       /* pa_validate_*: metadata contents are inconsistent */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Describes the two caller-owned device pools; see the conventions above. */
typedef struct {
    int32_t dtype;         /* pa_dtype                                           */
    int32_t num_blocks;    /* physical blocks in each pool                       */
    int32_t block_size;    /* B, tokens per block                                */
    int32_t num_kv_heads;  /* Hkv                                                */
    int32_t head_dim;      /* d                                                  */
    void* k_cache;         /* device, [num_blocks][B][Hkv][d]                    */
    void* v_cache;         /* device, same shape                                 */
} pa_kv_pool;

/* Human-readable name of a pa_status value (static string, never NULL). */
const char* pa_status_str(int status);

/* ABI version of this header (incremented on incompatible changes). */
int32_t pa_abi_version(void);

/* Digest of the sources the library was built from: 16 hex digits of a SHA-256 over
 * this header, every source of the package's csrc/ directory (relative path and bytes,
 * in name order) and the compile flags, as paged_kv_cache_73_amd/build.py computes it;
 * "unknown" for a build that did not pass it.  A static string, never freed.  It lets a
 * caller check that a prebuilt libpa.so matches the sources beside it. */
const char* pa_source_digest(void);

/* ---------------------------------------------------------------------------------
 * KV write ([QWEN] 自己来实现: one program per new token copies its HIDDEN_DIM K and V
 * values to row slot_mapping[n] of the cache and returns early for a negative slot).
 *
 * k_new, v_new: device, [num_tokens][Hkv][d], same dtype as the pool.
 * slot_mapping: device int32 [num_tokens]; slot = phys*B + offset.  Negative slots are
 *   skipped; slots >= num_blocks*B are skipped too (out of range).  Two tokens with
 *   the same non-negative slot is a caller error (the surviving row is unspecified).
 * The copy is bit-exact.  num_tokens == 0 is a no-op.
 * ------------------------------------------------------------------------------- */
int pa_write_kv(const pa_kv_pool* pool, const void* k_new, const void* v_new,
                const int32_t* slot_mapping, int32_t num_tokens, void* stream);

/* ---------------------------------------------------------------------------------
 * Copy-on-write data step ([PA11] §11.3: before writing into a shared block, allocate a
 * new block and copy the old contents there).  For i < num_pairs, block dst[i] of both
 * pools receives a bit-exact copy of block src[i].  src, dst: device int32 arrays; a
 * pair with an id outside [0, num_blocks) is skipped.  dst blocks must be distinct and
 * must not appear in src.  The pairs come from pa_bm_prepare_write.
 * ------------------------------------------------------------------------------- */
int pa_copy_blocks(const pa_kv_pool* pool, const int32_t* src, const int32_t* dst,
                   int32_t num_pairs, void* stream);

/* ---------------------------------------------------------------------------------
 * Decode: one query token per sequence ([HFPA] Çözme yolu; [QWEN] fast-attn 库的使用,
 * flash_attn_with_kvcache(q, k_cache, v_cache, cache_seqlens, block_table, scale)).
 *
 * out, q: device, [batch][num_heads][d], pool dtype.  out = softmax(scale * K q) V over
 *   the first seqlens_k[b] keys of sequence b, read through block_table row b.
 *   The KV of the current token must already be written (pa_write_kv), and
 *   seqlens_k counts it.  A sequence with no key gets a zero row.
 * block_table: device int32 [batch][max_blocks_per_seq].
 * seqlens_k: device int32 [batch], 0 <= seqlens_k[b] <= min(max_seqlen_k,
 *   max_blocks_per_seq*B).  Keys beyond max_blocks_per_seq*B are never read.
 * max_seqlen_k: host bound on seqlens_k, sizes the grid and the workspace.
 * partition_tokens: split-K partition length (a multiple of B), or 0 for an automatic
 *   choice from batch, num_kv_heads and max_seqlen_k (about seven workgroups per CU).
 *   It is rounded up to a multiple of max(B, 1024 / (2 * head_dim)), the keys one
 *   16-byte load per lane covers, which matters only for block_size 2 and 4.
 *   Keys are cut into partitions processed by different workgroups; each yields an
 *   online-softmax state (m, l, o) and a second kernel merges them with the [PA11]
 *   §11.2 rule.  Sequences with one partition are finished by the first kernel.
 * Large groups: bf16 pools with head_dim 64 or 128, B 16 or 32 and 5-8, 16 or 32 query
 *   heads per KV head run on the matrix-core kernel of pa_prefill_varlen (one query
 *   row per head, the group's heads sharing each key tile), with sequence offsets built
 *   from seqlens_k on the device; partition_tokens is then rounded up to whole 64-key
 *   tiles, and 0 plans key ranges of 16-32 tiles (or the whole sequence).  Such shapes
 *   always need a workspace, and softmax_scale must be positive and finite there
 *   (PA_ERR_INVALID_ARG otherwise), as for pa_prefill_varlen.
 * workspace: device scratch of at least pa_decode_workspace_bytes(...) bytes, called with
 *   the same batch, heads, head_dim, max_seqlen_k, partition_tokens and block size (may
 *   be NULL when that is 0; it covers either route, as the dtype is not an argument).  Its contents need no initialisation and are meaningless
 *   after the call; calls that share a workspace must not overlap.
 * Errors: PA_ERR_INVALID_ARG (null pointers, num_heads not a multiple of num_kv_heads,
 *   partition_tokens not a multiple of B), PA_ERR_WORKSPACE, PA_ERR_UNSUPPORTED (shape,
 *   batch > 65535).
 * ------------------------------------------------------------------------------- */
size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_seqlen_k,
                                 int32_t partition_tokens, int32_t block_size);

int pa_decode(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
              int32_t num_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
              const int32_t* seqlens_k, int32_t max_seqlen_k, float softmax_scale,
              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
              void* stream);

/* ---------------------------------------------------------------------------------
 * pa_decode_noalloc: pa_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  The split-K scratch is a static device array of the library,
 * PA_DECODE_SCRATCH_BYTES on each GPU it runs on, held until the process ends; the call
 * allocates nothing and frees nothing.  Arguments, results and the other errors as for
 * pa_decode.
 * Errors: PA_ERR_WORKSPACE when the call would need more scratch than the array holds
 *   (pa_decode_workspace_bytes(...) > PA_DECODE_SCRATCH_BYTES for these arguments),
 *   checked before any launch; PA_ERR_HIP when the array's address cannot be had.
 * Calls on one GPU share its array: calls that overlap on one GPU (other streams, other
 *   threads) race and must not be made; calls in order on one stream are fine.
 * ------------------------------------------------------------------------------- */
#define PA_DECODE_SCRATCH_BYTES (16u << 20)

int pa_decode_noalloc(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                      int32_t num_heads, const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* seqlens_k, int32_t max_seqlen_k, float softmax_scale,
                      int32_t partition_tokens, void* stream);

/* ---------------------------------------------------------------------------------
 * The two passes of pa_decode as separate calls (split-K decoding: partial states per
 * partition, then their merge by the [PA11] §11.2 rule), for callers that schedule
 * them apart or time them apart.  pa_decode_partials takes pa_decode's arguments plus
 * optional k_new, v_new (both NULL, or both given as for pa_decode_append); it finishes
 * the sequences that fit in one partition and leaves the others' partial states in the
 * workspace.  pa_decode_merge must follow on the same stream with the same pool, out,
 * batch, num_heads, max_blocks_per_seq, seqlens_k, max_seqlen_k, partition_tokens and
 * workspace (it reads the partials and writes the remaining rows; nothing to do when
 * no sequence was split).  pa_decode_partials then pa_decode_merge = pa_decode, bit
 * for bit.
 * ------------------------------------------------------------------------------- */
int pa_decode_partials(const pa_kv_pool* pool, void* out, const void* q, const void* k_new,
                       const void* v_new, int32_t batch, int32_t num_heads,
                       const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* seqlens_k, int32_t max_seqlen_k, float softmax_scale,
                       int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                       void* stream);
int pa_decode_merge(const pa_kv_pool* pool, void* out, int32_t batch, int32_t num_heads,
                    int32_t max_blocks_per_seq, const int32_t* seqlens_k, int32_t max_seqlen_k,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ---------------------------------------------------------------------------------
 * Decode with the KV write fused in ([HFPA] Çözme yolu: the decode kernel reads the cache
 * through block_table and updates it in place).  Same arguments and result as
 * pa_decode, plus k_new, v_new: device [batch][Hkv][d], the current token's K and V.
 * For each sequence with n = seqlens_k[b] >= 1 they are stored at position n-1 (block
 * block_table[b][(n-1)/B], slot (n-1)%B) and the n keys, that one included, are
 * attended.  The position's block must be private and assigned (pa_bm_prepare_write,
 * then pa_copy_blocks for its copy-on-write pairs); if its id is outside the pool the
 * row is neither stored nor attended.  Equivalent to pa_write_kv with those slots
 * followed by pa_decode, bit for bit (on the vector-unit kernel in one launch fewer; on
 * the large-group route the store is a small kernel of its own).
 * ------------------------------------------------------------------------------- */
int pa_decode_append(const pa_kv_pool* pool, void* out, const void* q, const void* k_new,
                     const void* v_new, int32_t batch, int32_t num_heads,
                     const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* seqlens_k, int32_t max_seqlen_k, float softmax_scale,
                     int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ---------------------------------------------------------------------------------
 * Varlen (packed) prefill with a paged cache ([QWEN] fast-attn 库的使用:
 * flash_attn_varlen_func(q, k_cache, v_cache, max_seqlen_q, cu_seqlens_q, max_seqlen_k,
 * cu_seqlens_k, scale, causal, block_table); [HFPA] Değişken uzunluklu yol).
 *
 * q, out: device, [total_q][num_heads][d] with total_q = cu_seqlens_q[batch], in the
 *   pool's dtype.  BF16 pools with block_size 16 or 32 and head_dim 64 or 128 run on the
 *   matrix cores; F32 pools, block_size 2, 4 or 8 and head_dim 256 run each query token as
 *   a decode query over its visible keys (no matrix cores, one partition per token).
 * cu_seqlens_q, cu_seqlens_k: device int32 [batch+1], non-decreasing from 0.  Request
 *   i owns query rows [cu_q[i], cu_q[i+1]) and k_len = cu_k[i+1]-cu_k[i] keys, read
 *   through block_table row i (only the differences of cu_k are used; the new tokens'
 *   K/V must already be written).  With c = k_len - q_len cached tokens, query row t
 *   sees keys j <= c + t when causal != 0 (bottom-right alignment), all k_len keys
 *   otherwise.  A row that sees no key gets zeros.
 * max_seqlen_q, max_seqlen_k: host bounds on the per-request lengths (grid sizing);
 *   queries of a request beyond max_seqlen_q are not computed.
 * softmax_scale must be positive and finite (PA_ERR_INVALID_ARG otherwise).
 * Supported: BF16 or F32 pools, head_dim 64 or 128, block_size 2, 4, 8, 16 or 32, group
 *   size num_heads / num_kv_heads from 1 to 8, 16 or 32, and on the token path
 *   num_kv_heads <= 64; head_dim 256 with block_size up to 16 (BF16) or 8 (F32).  On the
 *   token path group sizes 3, 5, 6, 7, 16 and 32 need head_dim 64 or 128 and block_size 8
 *   or more.  Otherwise PA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------------- */
int pa_prefill_varlen(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                      int32_t num_heads, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                      int32_t max_seqlen_k, const int32_t* block_table,
                      int32_t max_blocks_per_seq, float softmax_scale, int32_t causal,
                      void* stream);

/* ---------------------------------------------------------------------------------
 * Varlen prefill with key splitting: pa_prefill_varlen's result (the same masking,
 * alignment, shapes and errors) for batches with few query tiles.  On the matrix cores
 * a job (one request, KV head and tile of 128 query rows) walks all its keys in one
 * workgroup; when a batch has fewer jobs than the GPU has workgroup slots (a single long
 * prompt's chunk, a few requests with one query head per KV head), jobs are cut into
 * key ranges of at least 1024 keys processed by separate workgroups, each keeping the
 * online-softmax state (m, l, o) of its range ([PA11] §11.2), and a second kernel folds
 * the ranges with the §11.2 rule.  Results agree with pa_prefill_varlen within rounding
 * (bit-identical when nothing is split).
 *
 * host_cu_seqlens_q, host_cu_seqlens_k: optional HOST copies of the two cu_seqlens
 *   arrays (both or neither; NULL: plan from the bounds alone).  With them the split is
 *   planned from every job's key count (about one key range per workgroup slot); without
 *   them from max_seqlen_q and max_seqlen_k (for batches of mixed lengths the ranges are
 *   then longer than they need be).  Either way max_seqlen_q and max_seqlen_k must bound
 *   the requests' lengths; a request past max_seqlen_k still has all its keys attended
 *   (its last range takes the rest).
 * workspace: device scratch of at least pa_prefill_workspace_bytes(pool dtype, batch,
 *   num_heads, num_kv_heads, head_dim, block_size, max_seqlen_q, max_seqlen_k, causal,
 *   host_cu_seqlens_q, host_cu_seqlens_k) bytes, queried on the device the call runs on
 *   (the plan counts its CUs); NULL when that is 0: the batch has enough jobs, or the
 *   shape runs token by token.  Contents need no initialisation and are meaningless after
 *   the call; calls sharing a workspace must not overlap.
 * Errors: as pa_prefill_varlen, and PA_ERR_WORKSPACE when the workspace is missing or
 *   too small.
 * ------------------------------------------------------------------------------- */
size_t pa_prefill_workspace_bytes(int32_t dtype, int32_t batch, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t causal,
                                  const int32_t* host_cu_seqlens_q,
                                  const int32_t* host_cu_seqlens_k);

int pa_prefill_varlen_splitk(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                             int32_t num_heads, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                             int32_t max_seqlen_k, const int32_t* block_table,
                             int32_t max_blocks_per_seq, float softmax_scale, int32_t causal,
                             const int32_t* host_cu_seqlens_q, const int32_t* host_cu_seqlens_k,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Varlen prefill over contiguous (non-paged) K/V ([QWEN] fast-attn 库的使用: the same
 * varlen call without block_table, k and v then being packed like q; [HFPA]
 * Değişken uzunluklu yol).  The choice when nothing is cached yet.
 *
 * k, v: device, [total_k][num_kv_heads][head_dim] with total_k = cu_seqlens_k[batch];
 *   request i's keys are rows [cu_k[i], cu_k[i+1]).  q, out: [total_q][num_heads]
 *   [head_dim] as for pa_prefill_varlen; dtype PA_BF16 or PA_F32.  BF16 with head_dim 64
 *   or 128 runs on the matrix cores; F32 and head_dim 256 run each query token over its
 *   request's rows (the token path of pa_prefill_varlen), reading no key past
 *   max_seqlen_k.  Masking, alignment and scale as for pa_prefill_varlen; head_dim 64,
 *   128 or 256.  Nothing is owned or kept by the library.
 * ------------------------------------------------------------------------------- */
int pa_prefill_varlen_contiguous(void* out, const void* q, const void* k, const void* v,
                                 int32_t dtype, int32_t batch, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                                 int32_t causal, void* stream);

/* ---------------------------------------------------------------------------------
 * Measurement helper (not part of the attention path): reads `bytes` (a multiple of 16)
 * of device memory at `buf` with non-temporal 16-byte loads from `grid` workgroups of
 * 256 threads, each reading its own contiguous stretch, as a plain streaming read;
 * `sink` is a device word that is normally left untouched.  Timing it gives the attainable HBM read bandwidth that the decode
 * kernel is compared with.
 * ------------------------------------------------------------------------------- */
int pa_probe_stream_read(const void* buf, size_t bytes, void* sink, int32_t grid, void* stream);

/* =================================================================================
 * Host-side block manager and metadata builders (no device memory, single-threaded;
 * every pointer below is host memory).
 * ================================================================================= */

/* Reference-counted free stack of physical block ids ([PA11] §11.3: refs[p] counts the
 * block tables or prefix holders pointing at p; allocation sets 1, sharing adds 1,
 * release subtracts 1, and a block returns to the free stack only at 0; [NANO] 题目6:
 * free blocks are handed out 0, 1, 2, ... and a freed block is the next one reused). */
typedef struct pa_bm pa_bm;

/* initial_order: NULL for 0,1,2,..., else a permutation of [0, num_blocks) giving the
 * order in which blocks are first handed out.  *out receives the new manager. */
int pa_bm_create(int32_t num_blocks, const int32_t* initial_order, pa_bm** out);
void pa_bm_destroy(pa_bm* bm);
int32_t pa_bm_num_free(const pa_bm* bm);
/* Reference count of `block` (>= 0), or PA_ERR_INVALID_ARG for an id out of range. */
int pa_bm_refcount(const pa_bm* bm, int32_t block);
/* Copies the free stack, next-to-be-handed-out first, into out[0 .. *count). */
int pa_bm_free_stack(const pa_bm* bm, int32_t* out, int32_t capacity, int32_t* count);
/* Takes n blocks (refs = 1 each) into ids_out; all or nothing (PA_ERR_OUT_OF_BLOCKS). */
int pa_bm_alloc(pa_bm* bm, int32_t n, int32_t* ids_out);
int pa_bm_incref(pa_bm* bm, int32_t block);
/* Drops one reference; at 0 the block goes on top of the free stack. */
int pa_bm_decref(pa_bm* bm, int32_t block);
/* End of a request: drops one reference per assigned entry, walking the row in
 * reverse ([NANO] 题目6, deallocation). */
int pa_bm_release_table(pa_bm* bm, const int32_t* row, int32_t width);
/* Sharing: row_out = row, with one more reference on every assigned entry. */
int pa_bm_share(pa_bm* bm, const int32_t* row, int32_t width, int32_t* row_out);
/* Makes logical positions [start, start+count) of a table row writable: unassigned
 * entries get a new block ([NANO] 题目4, on-demand growth); entries whose block is
 * shared (refs > 1) get copy-on-write ([PA11] §11.3): a new block replaces the entry,
 * the old block loses this row's reference, and (src=old, dst=new) is appended to
 * cow_src/cow_dst (at most cow_capacity pairs; *num_cow receives the count).  All or
 * nothing: on PA_ERR_OUT_OF_BLOCKS neither the row nor the manager changes. */
int pa_bm_prepare_write(pa_bm* bm, int32_t block_size, int32_t* row, int32_t width,
                        int32_t start, int32_t count, int32_t* cow_src, int32_t* cow_dst,
                        int32_t cow_capacity, int32_t* num_cow);

/* Prefix cache ([NANO] 题目6: a block is looked up by compute_hash(token_ids, prefix_hash)
 * in hash_to_block_id; a hit adds a reference, a miss allocates; a freed block leaves the
 * map).  The page leaves compute_hash open; here it is FNV-1a 64 over the previous
 * block's hash (8 bytes, little-endian) followed by the block's token ids (4 bytes each,
 * little-endian), and the first block chains on 0. */
uint64_t pa_prefix_block_hash(const int32_t* tokens, int32_t n, uint64_t prefix_hash);
/* Table row for a request's n_tokens token ids: full block i is shared when its chained
 * hash is registered and the block holds the same token ids (one more reference),
 * otherwise a new block is taken and registered; the partial last block is always new
 * and unregistered.  row[width] receives the ids (-1 past the end); *n_hits (nullable)
 * the number of shared blocks, whose K/V need not be written again.  All or nothing
 * (PA_ERR_OUT_OF_BLOCKS).  Blocks freed by pa_bm_decref / pa_bm_release_table leave the
 * cache; a private registered block made writable by pa_bm_prepare_write leaves it too. */
int pa_bm_allocate_prefix(pa_bm* bm, int32_t block_size, const int32_t* tokens,
                          int32_t n_tokens, int32_t* row, int32_t width, int32_t* n_hits);

/* slots_out[i] = table[seq[i]][pos[i] / B] * B + pos[i] % B, or -1 when that entry is
 * unassigned ([QWEN] 自己来实现: slot_mapping is computed once and reused by every
 * layer).  table: [*][width]; PA_ERR_INVALID_ARG when pos[i]/B >= width or seq[i] < 0,
 * or when a slot would exceed INT32_MAX (slots are int32; nothing is written then). */
int pa_build_slot_mapping(const int32_t* table, int32_t width, int32_t block_size,
                          const int32_t* seq, const int32_t* pos, int32_t n,
                          int32_t* slots_out);
/* cu_out[0] = 0, cu_out[i+1] = cu_out[i] + lengths[i] ([HFPA] varlen example);
 * *max_out = max length (0 for batch 0). */
int pa_build_cu_seqlens(const int32_t* lengths, int32_t batch, int32_t* cu_out,
                        int32_t* max_out);

/* Pool bytes for K and V together ([PA11] §11.1: numBlocks * B * 2 * kvDim * elem). */
int64_t pa_pool_bytes(int32_t num_blocks, int32_t block_size, int32_t kv_dim,
                      int32_t elem_bytes);

/* Checks host copies of decode metadata: 0 <= seqlens[b] <= min(max_seqlen_k,
 * width*B) and every table entry a sequence's length reaches is in [0, num_blocks).
 * Returns PA_OK or PA_ERR_METADATA (*bad_index receives the first offending batch
 * row, may be NULL). */
int pa_validate_decode(const int32_t* table, int32_t batch, int32_t width,
                       const int32_t* seqlens, int32_t max_seqlen_k, int32_t num_blocks,
                       int32_t block_size, int32_t* bad_index);
/* Checks host copies of varlen metadata: cu arrays start at 0 and do not decrease,
 * q_len <= max_seqlen_q, k_len <= max_seqlen_k and k_len <= width*B, and table entries
 * reached are in range.  Note k_len < q_len is allowed (its first rows see nothing). */
int pa_validate_varlen(const int32_t* table, int32_t batch, int32_t width,
                       const int32_t* cu_q, const int32_t* cu_k, int32_t max_seqlen_q,
                       int32_t max_seqlen_k, int32_t num_blocks, int32_t block_size,
                       int32_t* bad_index);
/* Checks a slot mapping: every non-negative slot < num_blocks*B and no slot twice. */
int pa_validate_slots(const int32_t* slots, int32_t n, int32_t num_blocks,
                      int32_t block_size, int32_t* bad_index);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
