// Launch code of the varlen prefill kernel (prefill_kernel.h) and the merge of its
// key ranges, shared by the files that instantiate them (prefill_k128.hip,
// prefill_k128_odd.hip, prefill_k64.hip: the instantiations are spread over files so that
// they compile in parallel) and by prefill.hip, which plans and routes the calls.
#pragma once

#include <algorithm>
#include <atomic>

#include "prefill_kernel.h"

namespace pa {

// Where the keys live: a paged pool (table != null) or packed contiguous arrays.
struct KvSource {
    bool paged;
    const void* k;
    const void* v;
    int32_t num_kv_heads;
    int32_t num_blocks;   // paged only
    int32_t block_size;   // paged only
    const int32_t* table; // paged only
    int32_t max_blocks;   // paged only
};

struct SplitPlan {
    int32_t n_split;      // key ranges per job at most (1: no split)
    int32_t split_tiles;  // key tiles per range (the last range of a job takes the rest)
    int64_t units;        // dense jobs x n_split: rows of the workspace
};

// Second pass of a key-split prefill: for each row of a split job, the key ranges'
// states (m_s, l_s, O_s) are folded with the online-softmax merge ("Paged attention 与
// online softmax" §11.2: M = max m_s, O = sum 2^(m_s - M) O_s, l = sum 2^(m_s - M) l_s,
// in base 2 as the states are) and O / l is stored.  Jobs are indexed (request, KV head,
// query tile); jobs that were not split were finished by the first pass and are skipped.
// A workgroup takes kMergeRows rows of a job, a thread 4 dims of one row, and the
// ranges' loads are issued four at a time.
constexpr int kMergeThreads = 256;

template <int D, int G, int BS>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    uint16_t* __restrict__ out, int32_t num_heads, int32_t num_kv_heads, int32_t num_blocks,
    int32_t max_blocks, int32_t causal, int32_t n_qtiles, int32_t n_split, int32_t split_tiles,
    int32_t chunks, const float* __restrict__ part_o, const float2* __restrict__ part_ml) {
    constexpr int BN = kPrefillKeys;
    constexpr bool kPaged = BS > 0;
    constexpr int TOK = kPrefillRows / G;
    constexpr int D4 = D / 4;
    constexpr int kMergeRows = kMergeThreads / D4;       // rows per workgroup
    // chunks: workgroups per job, enough for the rows of min(TOK, max_seqlen_q) tokens
    const int64_t job = blockIdx.x / chunks;
    const int row = (blockIdx.x % chunks) * kMergeRows + threadIdx.x / D4;
    const int d4 = threadIdx.x % D4;
    const int qtile = static_cast<int>(job % n_qtiles);
    const int hkv = static_cast<int>((job / n_qtiles) % num_kv_heads);
    const int req = static_cast<int>(job / n_qtiles / num_kv_heads);
    const int q0 = cu_q[req];
    const int q_len = cu_q[req + 1] - q0;
    const int tok0 = qtile * TOK;
    const int tok = tok0 + row / G;
    if (tok >= q_len || row >= TOK * G) return;  // past the request, or an idle row
    // the first pass's key-tile count of this job, and so its number of key ranges
    const int k_len_req = cu_k[req + 1] - cu_k[req];
    const int k_len = kPaged ? min(k_len_req, max_blocks * BS) : k_len_req;
    const int tok_last = min(tok0 + TOK, q_len) - 1;
    const int kv_end = causal ? min(k_len, k_len_req - q_len + tok_last + 1) : k_len;
    const int n_tiles = (kv_end > 0 && (!kPaged || num_blocks > 0)) ? (kv_end + BN - 1) / BN : 0;
    const int parts = split_count(n_tiles, n_split, split_tiles);
    if (parts <= 1) return;
    const int64_t base = job * n_split * kPrefillRows + row;  // (range 0, this row)
    const float2* ml = part_ml + base;
    const float4* po = reinterpret_cast<const float4*>(part_o) + base * D4 + d4;
    float M = -INFINITY;
    for (int sp = 0; sp < parts; ++sp) M = fmaxf(M, ml[static_cast<int64_t>(sp) * kPrefillRows].x);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
    if (M != -INFINITY) {
        for (int sp0 = 0; sp0 < parts; sp0 += 4) {
            float2 st[4];
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t sp = min(sp0 + u, parts - 1);  // in range; the extra ones unused
                st[u] = ml[sp * kPrefillRows];
                v[u] = po[sp * kPrefillRows * D4];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (sp0 + u < parts) {
                    const float wgt = __builtin_amdgcn_exp2f(st[u].x - M);  // 0: empty range
                    L += wgt * st[u].y;
                    o.x += wgt * v[u].x;
                    o.y += wgt * v[u].y;
                    o.z += wgt * v[u].z;
                    o.w += wgt * v[u].w;
                }
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int head = hkv * G + row % G;
    uint16_t* orow = out + (static_cast<int64_t>(q0 + tok) * num_heads + head) * D + 4 * d4;
    const uint32_t lo = static_cast<uint32_t>(to_bf16_bits(o.x * inv)) |
                        (static_cast<uint32_t>(to_bf16_bits(o.y * inv)) << 16);
    const uint32_t hi = static_cast<uint32_t>(to_bf16_bits(o.z * inv)) |
                        (static_cast<uint32_t>(to_bf16_bits(o.w * inv)) << 16);
    *reinterpret_cast<uint2*>(orow) = make_uint2(lo, hi);
}

// The varlen prefill run token by token on the decode kernel (decode.hip): the path

// Workgroups of the prefill kernel that run at once: two per CU (LDS and registers),
// counted per device on first use.
inline int64_t prefill_slots() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int32_t> cus_of[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int cus = dev < kMaxDevices ? cus_of[dev].load(std::memory_order_relaxed) : 0;
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        if (dev < kMaxDevices) cus_of[dev].store(cus, std::memory_order_relaxed);
    }
    return 2 * static_cast<int64_t>(cus);
}

template <int D, int G, int BS>
int launch_prefill(const KvSource& kv, void* out, const void* q, int32_t batch,
                   int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                   int32_t max_seqlen_q, float scale, int32_t causal, hipStream_t stream,
                   const SplitPlan& sp, void* workspace, int passes) {
    const int tok_per_wg = kPrefillRows / G;
    const int64_t n_qtiles = (max_seqlen_q + tok_per_wg - 1) / tok_per_wg;
    const int64_t n_groups = static_cast<int64_t>(kv.num_kv_heads) * batch;
    const int64_t per_xcd = (n_groups + kXcds - 1) / kXcds * n_qtiles * sp.n_split;  // work units
    if (per_xcd * kXcds > INT32_MAX) return PA_ERR_UNSUPPORTED;
    const int32_t n_slots = static_cast<int32_t>(std::max<int64_t>(1, std::min(per_xcd, prefill_slots() / kXcds)));
    const int32_t cus_per_xcd = static_cast<int32_t>(prefill_slots() / (2 * kXcds));
    float* part_o = sp.n_split > 1 ? static_cast<float*>(workspace) : nullptr;
    float2* part_ml = sp.n_split > 1
        ? reinterpret_cast<float2*>(part_o + static_cast<size_t>(sp.units) * kPrefillRows * D) : nullptr;
    const dim3 grid(static_cast<uint32_t>(n_slots * kXcds));
    if (!(passes & kPass1)) {
        // the merge alone (of ranges stored by an earlier call)
    } else if (sp.n_split > 1)
        hipLaunchKernelGGL((prefill_kernel<D, G, BS, true>), grid, dim3(kPrefillThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const char*>(kv.k),
                           static_cast<const char*>(kv.v), cu_q, cu_k, kv.table,
                           static_cast<uint16_t*>(out), num_heads, kv.num_kv_heads,
                           kv.num_blocks, kv.max_blocks, scale * kLog2e, causal,
                           static_cast<int32_t>(n_qtiles), static_cast<int32_t>(n_groups),
                           sp.n_split, sp.split_tiles, part_o, part_ml, n_slots, cus_per_xcd);
    else
        hipLaunchKernelGGL((prefill_kernel<D, G, BS, false>), grid, dim3(kPrefillThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const char*>(kv.k),
                           static_cast<const char*>(kv.v), cu_q, cu_k, kv.table,
                           static_cast<uint16_t*>(out), num_heads, kv.num_kv_heads,
                           kv.num_blocks, kv.max_blocks, scale * kLog2e, causal,
                           static_cast<int32_t>(n_qtiles), static_cast<int32_t>(n_groups), 1, 0,
                           nullptr, nullptr, n_slots, cus_per_xcd);
    if (sp.n_split > 1 && (passes & kPass2)) {
        if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
        // workgroups per job: the rows of the tokens a query tile can hold (one token per
        // request in a decode step: G rows, not the tile's kPrefillRows)
        const int64_t merge_rows = kMergeThreads / (D / 4);
        const int64_t rows = static_cast<int64_t>(std::min(tok_per_wg, max_seqlen_q)) * G;
        const int64_t chunks = (rows + merge_rows - 1) / merge_rows;
        hipLaunchKernelGGL((prefill_merge_kernel<D, G, BS>), dim3(static_cast<uint32_t>(n_groups * n_qtiles * chunks)),
                           dim3(kMergeThreads), 0, stream, cu_q, cu_k, static_cast<uint16_t*>(out),
                           num_heads, kv.num_kv_heads, kv.num_blocks, kv.max_blocks, causal,
                           static_cast<int32_t>(n_qtiles), sp.n_split, sp.split_tiles,
                           static_cast<int32_t>(chunks),
                           static_cast<const float*>(part_o), static_cast<const float2*>(part_ml));
    }
    return launch_status();
}

// The launch of prefill_kernel<D, G, BS> for a group size G (one file per set of shapes).
#define PA_PREFILL_DISPATCH_ARGS                                                             \
    int G, const KvSource &kv, void *out, const void *q, int32_t batch, int32_t num_heads,   \
        const int32_t *cu_q, const int32_t *cu_k, int32_t max_seqlen_q, float scale,         \
        int32_t causal, hipStream_t stream, const SplitPlan &sp, void *workspace, int passes
int prefill_dispatch_k128(PA_PREFILL_DISPATCH_ARGS);      // G 1, 2, 4, 8
int prefill_dispatch_k128_odd(PA_PREFILL_DISPATCH_ARGS);  // G 3, 5, 6, 7, 16, 32
int prefill_dispatch_k64(PA_PREFILL_DISPATCH_ARGS);       // every G

}  // namespace pa

// Body of a dispatch function: the cases of the listed group sizes for head dim DD.
#define PA_PREFILL_LAUNCH(DD, GG, BB)                                                      \
    launch_prefill<DD, GG, BB>(kv, out, q, batch, num_heads, cu_q, cu_k, max_seqlen_q, scale, \
                               causal, stream, sp, workspace, passes)
#define PA_PREFILL_CASE(DD, GG)                                                            \
    case GG:                                                                               \
        if (!kv.paged) return PA_PREFILL_LAUNCH(DD, GG, 0);                                \
        return kv.block_size == 16 ? PA_PREFILL_LAUNCH(DD, GG, 16) : PA_PREFILL_LAUNCH(DD, GG, 32);
