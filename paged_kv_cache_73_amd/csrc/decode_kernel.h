#pragma once
// Paged decode attention: one query token per sequence, grouped-query heads,
// split-K over partitions of the context with an online-softmax merge.
//
// What it computes ("Sayfalı dikkat", Çözme yolu; "从零开始写Qwen3（六）PagedAttention",
// fast-attn 库的使用): out[b,h] = softmax(scale * K_b q[b,h]) V_b over the first
// seqlens[b] keys of sequence b, key p read from physical block table[b][p/B] at slot
// p mod B ("Paged attention 与 online softmax" §11.1).
//
// How (gfx950):
// * Pass 1, one workgroup per (sequence, partition, group of KV heads), one wave per
//   KV head.  A wave walks the pages of its partition; a page of one head is B rows of
//   d*elem bytes.  Lanes take consecutive 16-byte pieces of a row (LPR lanes cover a
//   row, so one load instruction covers 64/LPR whole rows = 1 KiB of the page), which
//   keeps every wave load fully coalesced; the workgroup as a whole streams whole
//   pages (B*Hkv*d contiguous elements) of K and then V.
// * The query heads that share the KV head (GQA group of G) are all served from the
//   same registers, so each K/V byte is read from HBM once.
// * QK dot products: each lane multiplies its 16 bytes, then DPP row permutations sum
//   the LPR lanes of a row.  Each lane keeps its own online-softmax state (m, l, o)
//   over the rows it loaded ("Paged attention 与 online softmax" §11.2: blocks of keys
//   can be folded in any grouping and merged), so P*V needs no cross-lane traffic.
//   At the end of the partition the row groups are merged with the same rule.
// * Softmax runs in base 2 (q is prescaled by scale*log2(e)), using the hardware exp2.
// * The next page's K and V are loaded before the current page is consumed, so two
//   pages per wave are in flight.
// * Pass 2 merges the partitions' (m, l, o) of every (sequence, head) with the boxed
//   rule of §11.2 and normalises.  A sequence that fits in one partition is finished
//   by pass 1 and skipped by pass 2.
// * Masked keys (past the sequence end, or in a block whose id is outside
//   [0, num_blocks)) are selected away, never multiplied by 0, and a block with an
//   invalid id is never loaded.

#include <algorithm>
#include <type_traits>

#include "common.h"

// Tuning knobs (compile time).  Heads per workgroup: how many KV heads (one wave each)
// share a workgroup; fewer means more, smaller workgroups and a shorter tail.
#ifndef PA_DECODE_HPW
#define PA_DECODE_HPW 2
#endif
// Occupancy hint: minimum waves per SIMD the register allocator must allow (0 = none).
#ifndef PA_DECODE_WAVES_PER_EU
#define PA_DECODE_WAVES_PER_EU 0
#endif
// Non-temporal K/V loads (the pages are streamed once).
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif

namespace pa {

// Cache policy of the K/V page loads: non-temporal (the pages are streamed once).
constexpr int32_t kLoadPolicy = PA_DECODE_NT ? 2 : 0;

template <typename T, int D, int BS>
struct PageShape {
    static constexpr int kElemBytes = Storage<T>::kBytes;
    static constexpr int kRowBytes = D * kElemBytes;
    static constexpr int kLanesPerRow = kRowBytes / 16;      // LPR
    static constexpr int kRowsPerLoad = kWave / kLanesPerRow;
    // Pages of fewer rows than one load covers (block size 2 or 4) are walked as "virtual
    // pages" of kRowsPerLoad keys, each lane loading its row from its own block.
    static constexpr bool kSmall = BS < kRowsPerLoad;
    static constexpr int kPagesPerStep = kSmall ? kRowsPerLoad / BS : 1;  // VP
    static constexpr int kStepKeys = BS * kPagesPerStep;     // keys per (virtual) page
    static constexpr int kLoads = kStepKeys / kRowsPerLoad;  // load instructions per page
    static constexpr int kElems = 16 / kElemBytes;           // values per lane per load
    static_assert(kLanesPerRow >= 1 && kLanesPerRow <= kWave, "row size");
    static_assert(kSmall ? kRowsPerLoad % BS == 0 : BS % kRowsPerLoad == 0,
                  "block size vs rows per load");
};

// Merge (m, l, o) with the state held by the lane `off` positions away (xor).
template <int E>
__device__ __forceinline__ void merge_xor(float& m, float& l, float (&o)[E], int off) {
    const float m_o = __shfl_xor(m, off);
    const float l_o = __shfl_xor(l, off);
    const float m_new = fmaxf(m, m_o);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float a = __builtin_amdgcn_exp2f(m - m_use);
    const float b = __builtin_amdgcn_exp2f(m_o - m_use);
    l = l * a + l_o * b;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float o_o = __shfl_xor(o[e], off);
        o[e] = o[e] * a + o_o * b;
    }
    m = m_new;
}

// Packed query tokens in place of sequences (the varlen prefill run token by token):
// "sequence" b is query token offset + blockIdx.z of the packed batch, its request is
// the one whose [cu_q[i], cu_q[i+1]) holds it, and it attends to that request's first
// k_len keys, or to keys j <= c + t when causal (c = k_len - q_len, t its index in the
// request).  cu_q == nullptr: ordinary decode.  With `contiguous`, the keys are packed
// rows (no block table): the pool has one row per block, and key j of request i is
// block cu_k[i] + j.
struct TokenMap {
    const int32_t* cu_q = nullptr;
    const int32_t* cu_k = nullptr;
    int32_t n_req = 0;
    int32_t causal = 0;
    int32_t offset = 0;
    int32_t max_q = 0;  // tokens of a request past max_q are not computed
    int32_t contiguous = 0;
};

#if PA_DECODE_WAVES_PER_EU > 0
#define PA_DECODE_ATTR __attribute__((amdgpu_waves_per_eu(PA_DECODE_WAVES_PER_EU)))
#else
#define PA_DECODE_ATTR
#endif

// G query heads per wave.  SPLIT > 1 spreads a KV head's group of G * SPLIT query heads
// over SPLIT waves (groups of 16 and 32, whose queries and states would not fit one
// wave's registers): each wave streams the KV head's pages for its own G heads, the
// pages being read again from L2 by the other waves of the group.
template <typename T, int D, int BS, int G, int SPLIT = 1>
__global__ __launch_bounds__(PA_DECODE_HPW * kWave) PA_DECODE_ATTR void decode_partial_kernel(
    const T* __restrict__ q, char* k_cache, char* v_cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    const T* __restrict__ k_new, const T* __restrict__ v_new,
    T* __restrict__ out, float* __restrict__ o_part, float* __restrict__ ml_part,
    int32_t num_heads, int32_t num_kv_heads, int32_t num_blocks, int32_t max_blocks,
    int32_t max_parts, int32_t part_pages, float qscale, TokenMap tm) {
    using S = PageShape<T, D, BS>;
    constexpr int LPR = S::kLanesPerRow;
    constexpr int RPL = S::kRowsPerLoad;
    constexpr int NL = S::kLoads;
    constexpr int VP = S::kPagesPerStep;  // pages per step (1 unless pages are small)
    constexpr int SK = S::kStepKeys;      // keys per step
    constexpr int E = S::kElems;

    const int lane = threadIdx.x % kWave;
    const int heads_per_wg = blockDim.x / kWave;
    const int vkv = blockIdx.x * heads_per_wg + threadIdx.x / kWave;  // wave of the grid
    const int hkv = vkv / SPLIT;                  // its KV head
    const int h0 = hkv * (G * SPLIT) + (vkv % SPLIT) * G;  // its first query head
    const int part = blockIdx.y;
    const int b = blockIdx.z + tm.offset;
    const int r0 = lane / LPR;  // first row of this lane within a load
    const int c = lane % LPR;   // 16-byte piece of the row

    const int32_t cap = max_blocks * BS;
    int32_t n_keys;
    int64_t row_index = b;  // block-table row
    int32_t first_block = 0;  // contiguous keys: the block (row) of key 0
    if (tm.cu_q != nullptr) {
        if (b >= tm.cu_q[tm.n_req]) return;  // past the packed tokens (uniform)
        int lo = 0, hi = tm.n_req;           // cu_q[lo] <= b < cu_q[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tm.cu_q[mid] <= b) lo = mid; else hi = mid;
        }
        const int32_t q_len = tm.cu_q[lo + 1] - tm.cu_q[lo];
        const int32_t k_len = tm.cu_k[lo + 1] - tm.cu_k[lo];
        const int32_t t = b - tm.cu_q[lo];
        if (t >= tm.max_q) return;
        n_keys = tm.causal ? min(k_len, k_len - q_len + t + 1) : k_len;
        row_index = lo;
        if (tm.contiguous) first_block = tm.cu_k[lo];
    } else {
        n_keys = seqlens[b];
    }
    const int32_t seqlen = min(max(n_keys, 0), cap);
    const int32_t part_tokens = part_pages * BS;
    const int32_t n_parts = max(1, (seqlen + part_tokens - 1) / part_tokens);
    // uniform over the workgroup; the grid may hold one row past max_parts (odd row count)
    if (part >= n_parts || part >= max_parts) return;
    const int32_t t_end = min(seqlen, (part + 1) * part_tokens);
    const int32_t pg0 = part * part_pages;
    int32_t pg1 = (t_end + BS - 1) / BS;

    // query heads of this KV head, this lane's E dims, prescaled to base 2
    float qv[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int h = h0 + g;
        const uint4 w = *reinterpret_cast<const uint4*>(
            q + (static_cast<int64_t>(b) * num_heads + h) * D + c * E);
        widen(w, qv[g], T{});
#pragma unroll
        for (int e = 0; e < E; ++e) qv[g][e] *= qscale;
    }

    // Fused append (k_new != null): the current token sits at position seqlen - 1.  The
    // workgroup of the last partition stores its K/V row in the cache and, when it
    // consumes that page, takes the row from registers rather than from memory.
    const int32_t* table_row = tm.contiguous ? nullptr : block_table + row_index * max_blocks;
    const bool appending = k_new != nullptr && seqlen > 0 && part == n_parts - 1;
    const int32_t new_pos = seqlen - 1;
    uint4 nk = make_uint4(0, 0, 0, 0), nv = make_uint4(0, 0, 0, 0);
    if (appending) {
        const int64_t nrow = (static_cast<int64_t>(b) * num_kv_heads + hkv) * D + c * E;
        nk = *reinterpret_cast<const uint4*>(k_new + nrow);
        nv = *reinterpret_cast<const uint4*>(v_new + nrow);
        const int32_t id = table_row[new_pos / BS];
        if (r0 == 0 && id >= 0 && id < num_blocks && vkv % SPLIT == 0) {  // one wave of the group
            const int64_t off = ((static_cast<int64_t>(id) * BS + new_pos % BS) * num_kv_heads + hkv) *
                                    S::kRowBytes + c * 16;
            *reinterpret_cast<uint4*>(k_cache + off) = nk;
            *reinterpret_cast<uint4*>(v_cache + off) = nv;
        }
    }

    float m[G], l[G], o[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] = 0.f;
    }

    const int32_t page_bytes = BS * num_kv_heads * S::kRowBytes;
    // byte offset of this lane's first piece inside a page, and the step between loads
    const int32_t lane_off = (r0 * num_kv_heads + hkv) * S::kRowBytes + c * 16;
    const int32_t load_step = RPL * num_kv_heads * S::kRowBytes;

    // Consume one page of K/V already in registers.  A page whose block id is outside
    // [0, num_blocks) was loaded from block 0 instead and is masked entirely.  Values are
    // widened to fp32 one 16-byte piece at a time to keep few registers live.
    // With small pages the id is this lane's own block and every row is checked.
    auto consume = [&](int32_t id, int32_t tok0, const uint4 (&kb)[NL], const uint4 (&vb)[NL]) {
        const bool valid = id >= 0 && id < num_blocks;
        const bool partial = S::kSmall || !valid || tok0 + SK > t_end;
        const bool has_new = appending && tok0 + SK > new_pos;  // uniform: the last page
        auto piece = [&](const uint4 (&buf)[NL], const uint4& fresh, int j) {
            uint4 x = buf[j];
            if (has_new && tok0 + r0 + j * RPL == new_pos) x = fresh;
            return x;
        };
        float s[G][NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            float kf[E];
            widen(piece(kb, nk, j), kf, T{});
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) acc += qv[g][e] * kf[e];
                s[g][j] = group_sum<LPR>(acc);
            }
        }
        bool ok[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) ok[j] = !partial || (valid && tok0 + r0 + j * RPL < t_end);
        if (partial) {
#pragma unroll
            for (int j = 0; j < NL; ++j)
#pragma unroll
                for (int g = 0; g < G; ++g) s[g][j] = ok[j] ? s[g][j] : -INFINITY;
        }
        // online-softmax update of this lane's state with its NL rows
        float p[G][NL];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = s[g][0];
#pragma unroll
            for (int j = 1; j < NL; ++j) mx = fmaxf(mx, s[g][j]);
            const float m_new = fmaxf(m[g], mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // nothing seen yet
            const float corr = __builtin_amdgcn_exp2f(m[g] - m_use);
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                p[g][j] = __builtin_amdgcn_exp2f(s[g][j] - m_use);
                psum += p[g][j];
            }
            l[g] = l[g] * corr + psum;
            m[g] = m_new;
#pragma unroll
            for (int e = 0; e < E; ++e) o[g][e] *= corr;
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            float vf[E];
            widen(piece(vb, nv, j), vf, T{});
            if (partial) {  // a masked row may hold anything (NaN): select, never multiply
#pragma unroll
                for (int e = 0; e < E; ++e) vf[e] = ok[j] ? vf[e] : 0.f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < E; ++e) o[g][e] += p[g][j] * vf[e];
        }
    };
    // Issue the loads of one page through a buffer descriptor spanning exactly that
    // page: one 32-bit lane offset, the row step in the scalar offset, and accesses the
    // hardware bounds-checks against the page.  Invalid ids read block 0 instead.
    auto load_page = [&](int32_t id, uint4 (&kd)[NL], uint4 (&vd)[NL]) {
        if constexpr (S::kSmall) {  // one row per lane group, each from its own block
            const int64_t at = static_cast<int64_t>((id >= 0 && id < num_blocks) ? id : 0) * page_bytes +
                               ((r0 % BS) * num_kv_heads + hkv) * S::kRowBytes + c * 16;
            kd[0] = *reinterpret_cast<const uint4*>(k_cache + at);
            vd[0] = *reinterpret_cast<const uint4*>(v_cache + at);
            return;
        }
        const int64_t base = static_cast<int64_t>((id >= 0 && id < num_blocks) ? id : 0) * page_bytes;
        const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(k_cache + base), 0, static_cast<int32_t>(page_bytes), kBufferDword3);
        const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(v_cache + base), 0, static_cast<int32_t>(page_bytes), kBufferDword3);
#pragma unroll
        for (int j = 0; j < NL; ++j) kd[j] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(kr, lane_off, j * load_step, kLoadPolicy));
#pragma unroll
        for (int j = 0; j < NL; ++j) vd[j] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(vr, lane_off, j * load_step, kLoadPolicy));
    };

    if (num_blocks <= 0) pg1 = pg0;  // nothing can be read
    for (int32_t pc = pg0; pc < pg1; pc += kWave) {
        const int np = (min(kWave, pg1 - pc) + VP - 1) / VP;  // (virtual) pages of the chunk
        const int32_t my_id = lane >= min(kWave, pg1 - pc) ? -1
                              : tm.contiguous ? first_block + pc + lane : table_row[pc + lane];
        // id of step i: a scalar, or with small pages this lane's block
        auto step_id = [&](int i) -> int32_t {
            if constexpr (S::kSmall) return __shfl(my_id, i * VP + r0 / BS);
            else return __builtin_amdgcn_readlane(my_id, i);
        };
        // ping-pong: while one page is consumed the next one is in flight
        uint4 ka[NL], va[NL], kb[NL], vb[NL];
        int32_t id_a = step_id(0);
        load_page(id_a, ka, va);
        int i = 0;
        for (; i + 2 < np; i += 2) {
            const int32_t id_b = step_id(i + 1);
            load_page(id_b, kb, vb);
            consume(id_a, (pc + i * VP) * BS, ka, va);
            id_a = step_id(i + 2);
            load_page(id_a, ka, va);
            consume(id_b, (pc + (i + 1) * VP) * BS, kb, vb);
        }
        if (i + 1 < np) {
            const int32_t id_b = step_id(i + 1);
            load_page(id_b, kb, vb);
            consume(id_a, (pc + i * VP) * BS, ka, va);
            consume(id_b, (pc + (i + 1) * VP) * BS, kb, vb);
        } else {
            consume(id_a, (pc + i * VP) * BS, ka, va);
        }
    }

    // merge the row groups (lanes with the same piece c)
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) merge_xor<E>(m[g], l[g], o[g], off);
    }
    if (r0 != 0) return;

#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int h = h0 + g;
        const int64_t bh = static_cast<int64_t>(b) * num_heads + h;
        if (n_parts == 1) {
            float r[E];
            const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) r[e] = o[g][e] * inv;
            *reinterpret_cast<uint4*>(out + bh * D + c * E) = narrow(r, T{});
        } else {
            float* op = o_part + (bh * max_parts + part) * D + c * E;
#pragma unroll
            for (int e = 0; e < E; e += 4)
                *reinterpret_cast<float4*>(op + e) = make_float4(o[g][e], o[g][e + 1], o[g][e + 2], o[g][e + 3]);
            if (c == 0)
                *reinterpret_cast<float2*>(ml_part + (bh * max_parts + part) * 2) = make_float2(m[g], l[g]);
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(
    const int32_t* __restrict__ seqlens, const float* __restrict__ o_part,
    const float* __restrict__ ml_part, T* __restrict__ out, int32_t num_heads, int32_t cap,
    int32_t max_parts, int32_t part_tokens) {
    constexpr int PER = D / kWave;    // dims per lane
    constexpr int CH = 32 / PER;      // partitions whose o rows are loaded together
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int64_t bh = static_cast<int64_t>(b) * num_heads + h;
    const float2* ml = reinterpret_cast<const float2*>(ml_part) + bh * max_parts;
    const float* op = o_part + bh * max_parts * D;

    // Loads that do not depend on the sequence length go out first, together with it: the
    // (m, l) of partitions 0..63 and the o rows of the first CH partitions, at indices
    // clamped to the workspace (entries past the sequence's partitions are never used:
    // they are selected away, not multiplied, since the workspace there is uninitialised).
    const int32_t seqlen_raw = seqlens[b];
    const int last = max_parts - 1;
    const float2 st = ml[min(lane, last)];
    float v[CH][PER];
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
        for (int k = 0; k < PER; ++k) v[u][k] = op[min(u, last) * D + lane + k * kWave];
    // keep the compiler from sinking these loads below the length test (it would wait for
    // the length first and then for the loads: two trips to memory instead of one)
    asm volatile("" ::"v"(st.x), "v"(st.y));
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
        for (int k = 0; k < PER; ++k) asm volatile("" ::"v"(v[u][k]));
    const int32_t seqlen = min(max(seqlen_raw, 0), cap);
    const int32_t n_parts = max(1, (seqlen + part_tokens - 1) / part_tokens);
    if (n_parts == 1) return;  // finished by pass 1

    float L = 0.f, O[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) O[k] = 0.f;
    // Lane p of block b holds the state of partition 64b + p.  The global maximum first;
    // then per block of 64 partitions the weights and l, and the o rows CH partitions at
    // a time, the next CH (the next block's first ones at a block's end) in flight while
    // the current ones are summed.  Partitions are summed in order.
    float M = lane < n_parts ? st.x : -INFINITY;
    for (int p = lane + kWave; p < n_parts; p += kWave) M = fmaxf(M, ml[p].x);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (M != -INFINITY) {
        for (int p0 = 0; p0 < n_parts; p0 += kWave) {
            const int cnt = min(kWave, n_parts - p0);
            const bool mine = lane < cnt;
            const float2 sp = p0 == 0 ? st : ml[min(p0 + lane, last)];
            const float wl = mine ? __builtin_amdgcn_exp2f(sp.x - M) : 0.f;
            L += mine ? wl * sp.y : 0.f;
            for (int c0 = 0;; c0 += CH) {
                const int nx = c0 + CH < cnt ? p0 + c0 + CH : p0 + kWave;  // next chunk
                const bool more = nx < n_parts;
                float vn[CH][PER];
                if (more) {
#pragma unroll
                    for (int u = 0; u < CH; ++u)
#pragma unroll
                        for (int k = 0; k < PER; ++k)
                            vn[u][k] = op[min(nx + u, last) * D + lane + k * kWave];
                }
#pragma unroll
                for (int u = 0; u < CH; ++u) {
                    if (c0 + u < cnt) {
                        const float w = __int_as_float(
                            __builtin_amdgcn_readlane(__float_as_int(wl), c0 + u));
#pragma unroll
                        for (int k = 0; k < PER; ++k) O[k] += w * v[u][k];
                    }
                }
                if (more) {
#pragma unroll
                    for (int u = 0; u < CH; ++u)
#pragma unroll
                        for (int k = 0; k < PER; ++k) v[u][k] = vn[u][k];
                }
                if (c0 + CH >= cnt) break;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const float r = O[k] * inv;
        if constexpr (sizeof(T) == 4) {
            out[bh * D + lane + k * kWave] = r;
        } else {
            reinterpret_cast<uint16_t*>(out)[bh * D + lane + k * kWave] = to_bf16_bits(r);
        }
    }
}

template <typename T, int D, int BS, int G, int SPLIT = 1>
int launch_decode(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                  int32_t num_heads, const int32_t* table, int32_t max_blocks,
                  const int32_t* seqlens, const void* k_new, const void* v_new, int32_t max_parts,
                  int32_t part_tokens, float scale, float* o_part, float* ml_part, hipStream_t stream,
                  const TokenMap& tm, int passes) {
    const int hkv = pool->num_kv_heads;
    const int waves = hkv * SPLIT;  // one wave per KV head and split of its group
    int per_wg = PA_DECODE_HPW;
    while (waves % per_wg != 0) per_wg >>= 1;
    // Workgroups go to the 8 XCDs round-robin in launch order.  With an even number of
    // partition rows, partition p of every sequence would land on the same XCDs (those of
    // p's parity), and the XCDs holding the later, partial or absent partitions would run
    // short of work; an odd row count (an empty row added) rotates the assignment from one
    // sequence to the next.
    const dim3 grid(waves / per_wg, max_parts | 1, batch);
    if (passes & kPass1) hipLaunchKernelGGL((decode_partial_kernel<T, D, BS, G, SPLIT>), grid, dim3(per_wg * kWave), 0, stream,
                       static_cast<const T*>(q), static_cast<char*>(pool->k_cache),
                       static_cast<char*>(pool->v_cache), table, seqlens,
                       static_cast<const T*>(k_new), static_cast<const T*>(v_new),
                       static_cast<T*>(out), o_part, ml_part, num_heads, hkv, pool->num_blocks,
                       max_blocks, max_parts, part_tokens / BS, scale * kLog2e, tm);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    if ((passes & kPass2) && max_parts > 1) {
        hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(num_heads, batch), dim3(kWave), 0,
                           stream, seqlens, o_part, ml_part, static_cast<T*>(out), num_heads,
                           max_blocks * BS, max_parts, part_tokens);
    }
    return launch_status();
}

// Group sizes 1, 2, 4 and 8 are instantiated in decode.hip; 3, 5, 6, 7, 16 and 32 in
// decode_groups.hip (for the shapes listed there), so the two compile in parallel.
template <typename T, int D, int BS>
int dispatch_group_pow2(int G, const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                   int32_t num_heads, const int32_t* table, int32_t max_blocks,
                   const int32_t* seqlens, const void* k_new, const void* v_new, int32_t max_parts,
                   int32_t part_tokens, float scale, float* o_part, float* ml_part,
                   hipStream_t stream, const TokenMap& tm, int passes) {
#define PA_DECODE_G(GG)                                                                    \
    case GG:                                                                               \
        return launch_decode<T, D, BS, GG>(pool, out, q, batch, num_heads, table, max_blocks, \
                                           seqlens, k_new, v_new, max_parts, part_tokens,    \
                                           scale, o_part, ml_part, stream, tm, passes);
    switch (G) {
        PA_DECODE_G(1)
        PA_DECODE_G(2)
        PA_DECODE_G(4)
        PA_DECODE_G(8)
        default: return PA_ERR_UNSUPPORTED;
    }
#undef PA_DECODE_G
}

template <typename T, int D, int BS>
int dispatch_group_odd(int G, const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                   int32_t num_heads, const int32_t* table, int32_t max_blocks,
                   const int32_t* seqlens, const void* k_new, const void* v_new, int32_t max_parts,
                   int32_t part_tokens, float scale, float* o_part, float* ml_part,
                   hipStream_t stream, const TokenMap& tm, int passes) {
#define PA_DECODE_G(GG)                                                                    \
    case GG:                                                                               \
        return launch_decode<T, D, BS, GG>(pool, out, q, batch, num_heads, table, max_blocks, \
                                           seqlens, k_new, v_new, max_parts, part_tokens,    \
                                           scale, o_part, ml_part, stream, tm, passes);
    switch (G) {
        PA_DECODE_G(3)
        PA_DECODE_G(5)
        PA_DECODE_G(6)
        PA_DECODE_G(7)
        case 16:
            return launch_decode<T, D, BS, 8, 2>(pool, out, q, batch, num_heads, table, max_blocks,
                                                 seqlens, k_new, v_new, max_parts, part_tokens,
                                                 scale, o_part, ml_part, stream, tm, passes);
        case 32:
            return launch_decode<T, D, BS, 8, 4>(pool, out, q, batch, num_heads, table, max_blocks,
                                                 seqlens, k_new, v_new, max_parts, part_tokens,
                                                 scale, o_part, ml_part, stream, tm, passes);
        default: return PA_ERR_UNSUPPORTED;
    }
#undef PA_DECODE_G
}

}  // namespace pa
