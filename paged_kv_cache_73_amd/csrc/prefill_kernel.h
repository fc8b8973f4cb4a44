// Varlen (packed) paged prefill on the matrix cores: the kernel.
//
// What it computes ("从零开始写Qwen3（六）PagedAttention", fast-attn 库的使用: the varlen call
// with a block table; "Sayfalı dikkat", Değişken uzunluklu yol): request i owns query
// rows [cu_q[i], cu_q[i+1]) of the packed q and k_len = cu_k[i+1] - cu_k[i] keys, read
// through block_table row i ("Paged attention 与 online softmax" §11.1).  With
// c = k_len - q_len cached tokens, query row t sees keys j <= c + t when causal.
//
// How (gfx950, bf16 in, fp32 accumulate):
// * A job is 128 "rows" of one request and one KV head, a row being a (token, query
//   head) pair with the G query heads of the KV head next to each other, so every K/V
//   tile read serves all of them.  A workgroup of four waves (32 rows each) runs a list of
//   jobs; two workgroups per CU put two waves on every SIMD.  A single wave issues at
//   most one instruction every fourth cycle, which, with the softmax, the loads and the
//   operand reads beside its products, would leave the matrix core idle half the time; a
//   second wave issues while the first waits.  (The register file then holds 32 rows of
//   O per wave, and each K or V^T operand read from LDS feeds one product.)
// * Keys are walked in tiles of 32, FlashAttention-style ("结合nanovllm的FlashAttention和
//   PagedAttention主要原理概述" 题目3): each tile is gathered through the block table into LDS,
//   its scores are folded into the running (m, l, O) with the §11.2 rule, and O is
//   normalised once at the end.
// * Transposed products keep a query row inside one lane: S^T = K Q^T with
//   v_mfma_f32_32x32x16_bf16 (A = a K row per lane from LDS, B = the lane's q row held in
//   registers), so lane l holds 16 of the tile's scores for row l%32 (the other 16 sit in
//   lane l^32).  O^T += V^T P^T takes P straight from the S^T accumulators; its V^T
//   operand comes from V stored as it is in memory (key-major) through gfx950's
//   transposing LDS read, in the key order in which the accumulators hold the weights.
// * K and V tiles go from memory to LDS by direct loads (no registers, no LDS stores):
//   each wave loads an 8-key slice of every tile, which lies in one page, so the page
//   address is a scalar; loads bounded to the slice's valid keys return zeros past kv_end
//   and for a block id outside the pool, so masked keys never bring NaN into a product.
//   Masking sets scores past a row's limit (and of unassigned blocks) to -inf.
// * Software pipeline, one barrier per tile, each step in two phases: the step's 16
//   products back to back at raised wave priority (tile t+1's scores, then tile t's P V
//   with the weights made the step before), then tile t+1's weights on the vector unit at
//   normal priority.  The other wave of the SIMD (another workgroup) runs its products
//   while this one does its vector work, and the matrix core they share makes them take
//   turns.  Four LDS stages: t (V read), t+1 (K read), and the loads of t+2 and t+3 in
//   flight, two steps ahead of their use.
// * The start of a launch: cu_seqlens go to LDS once, the workgroups work out the same
//   orders of requests and units (longest first) there, and meanwhile pull the q rows
//   of their XCD into its L2.  The unit lists are then placed on the CUs by load: two
//   workgroups that share a CU share its SIMDs, so each CU pairs a heavy list with a
//   light one.
// * The end of a unit: O goes through LDS (a K stage per wave) so that the stores write
//   whole 16-byte pieces of each output row.
// * Weights without a per-tile maximum: p = 2^(s*scale*log2e - m) against the row's
//   reference m, the row's maximum over the unit's first tile.  The quotient
//   sum(p v) / sum(p) does not depend on m; a tile whose weights sum past 2^64 sends the
//   unit down a slow path that recomputes it against exact row maxima.  Row sums are taken
//   from the bf16 weights that enter the products (v_dot2).
// * BS = 0 instantiates the same kernel for contiguous K/V (the varlen call without a
//   block table): request i's keys are rows [cu_k[i], cu_k[i+1]) of packed
//   [sum_k][Hkv][d] arrays, and only the loader's addressing differs.
#pragma once

#include <type_traits>

#include "common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4_ptr_t;

template <int S> using Stage = std::integral_constant<int, S>;

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, const uint16_t* dst,
                                           int32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(dst)), 16, voffset, 0, 0, 0);
}

// 4 bytes per lane: lane l's bytes land at dst + 4 l
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t rsrc, const uint16_t* dst,
                                          int32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(dst)), 4, voffset, 0, 0, 0);
}

__device__ __forceinline__ lds_v4_ptr_t to_lds_v4(const uint16_t* p) {
    return (lds_v4_ptr_t)(const_cast<uint16_t*>(p));
}

// Wait until at most N of this wave's vector-memory instructions are outstanding (they
// complete in order), then the workgroup barrier.  Direct-to-LDS loads count there, so
// a wave's own loads of a stage have landed once it passes; the barrier makes them
// every wave's.  The compiler's own barrier would first wait for every load in flight;
// this one keeps the later stages' loads flying.  (The memory clobber keeps LDS accesses
// on their side of it.)
// A barrier after this wave's LDS accesses only: loads from memory may stay in flight
// (the workgroup barrier of the language waits for them too).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

constexpr int kRowBlocks = 1;                            // 32-row blocks per wave
constexpr int kWaveRows = 32 * kRowBlocks;                // rows per wave
constexpr int kPrefillRows = 128;                         // rows per workgroup (a job)
constexpr int kPrefillWaves = kPrefillRows / kWaveRows;   // waves per workgroup
constexpr int kWavesPerSimd = 2 / kRowBlocks;             // resident waves per SIMD
constexpr int kPrefillKeys = 32;                          // keys per tile
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kPrefillStages = 4;                         // LDS tile buffers
constexpr int kXcds = 8;            // accelerator complex dies of an MI355X
constexpr float kFastSumLimit = 18446744073709551616.f;  // 2^64: weights of a tile on the fast path
constexpr int kMaxRankedRequests = 256;
constexpr int64_t kQPrefetchBytes = 3 << 20;  // at most this much of q per XCD is pulled into L2 at the start  // requests ordered by key count in-kernel
// Jobs per XCD ordered by key tiles in-kernel.  Ranking costs O(jobs^2) LDS compares per
// workgroup and separates the query tiles of a group (which then stop sharing K/V pages
// in L2); past a few jobs per workgroup slot the batch order, which keeps a group's tiles
// together, measured faster.
constexpr int kMaxRankedJobs = 384;
// Most workgroups per XCD whose lists are placed on the CUs by their load (below); a
// larger grid keeps the plain deal.
constexpr int kMaxPlacedSlots = 64;
// What starting a unit costs its slot, in key tiles (its first loads, q rows, the store):
// ~2 us against ~1 us per tile when two workgroups share a CU.
constexpr int kUnitCostTiles = 2;

// Key ranges of a job of `tiles` key tiles when jobs are cut into ranges of split_tiles
// tiles, at most n_split of them (the last one takes the rest).
__host__ __device__ inline int split_count(int tiles, int n_split, int split_tiles) {
    if (n_split <= 1 || tiles <= split_tiles) return 1;
    const int parts = (tiles + split_tiles - 1) / split_tiles;
    return parts < n_split ? parts : n_split;
}

constexpr bf16x2_t kOnes2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

// BS = 0: contiguous K/V.  kSplit: jobs may be cut into key ranges (n_split, split_tiles);
// without it those arguments are ignored and the kernel is the plain one.
template <int D, int G, int BS, bool kSplit>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd))) void prefill_kernel(
    const uint16_t* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ block_table,
    uint16_t* __restrict__ out, int32_t num_heads, int32_t num_kv_heads, int32_t num_blocks,
    int32_t max_blocks, float qscale, int32_t causal, int32_t n_qtiles, int32_t n_groups,
    int32_t n_split_arg, int32_t split_tiles_arg, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int32_t n_slots, int32_t cus_per_xcd) {
    const int n_split = kSplit ? n_split_arg : 1;
    const int split_tiles = kSplit ? split_tiles_arg : 0;
    constexpr int BN = kPrefillKeys;
    constexpr bool kPaged = BS > 0;
    constexpr int PBS = kPaged ? BS : BN;       // keys per page (one page per tile when contiguous)
    constexpr int PAGES = BN / PBS;             // pages of a tile (1 or 2)
    constexpr int TOK = kPrefillRows / G;       // tokens per workgroup
    constexpr int KS = D / 16;                  // MFMA k-steps over the head dim
    constexpr int DB = D / 32;                  // 32-wide blocks of the head dim in O^T
    constexpr int RB = kRowBlocks;
    constexpr int NP = 8 * RB;                  // weight pairs per lane and tile
    constexpr int CHUNKS = D / 8;               // 16-byte pieces per K/V row
    constexpr int SLICE = BN / kPrefillWaves;   // keys of a tile loaded by each wave
    static_assert(D == 64 || D == 128, "head dims");
    static_assert(PBS % SLICE == 0 && BN % PBS == 0, "a wave's keys lie in one page");
    // LDS: four stages of a K and a V tile (BN key-major rows of D elements each), each
    // its own array, so that the compiler's wait counts can tell the stages' loads apart
    constexpr int TILE = BN * D;
    static_assert(kPrefillStages == 4, "four stages");
    __shared__ __align__(16) uint16_t k_st0[TILE], k_st1[TILE], k_st2[TILE], k_st3[TILE];
    __shared__ __align__(16) uint16_t v_st0[TILE], v_st1[TILE], v_st2[TILE], v_st3[TILE];
    auto k_of = [&](auto st) -> uint16_t* {
        constexpr int S = decltype(st)::value;
        if constexpr (S == 0) return k_st0; else if constexpr (S == 1) return k_st1;
        else if constexpr (S == 2) return k_st2; else return k_st3;
    };
    auto v_of = [&](auto st) -> uint16_t* {
        constexpr int S = decltype(st)::value;
        if constexpr (S == 0) return v_st0; else if constexpr (S == 1) return v_st1;
        else if constexpr (S == 2) return v_st2; else return v_st3;
    };
    static_assert((kMaxRankedRequests + kMaxRankedJobs) * 4 <= TILE * 2 && kMaxRankedJobs * 4 <= TILE * 2,
                  "the ranking's scratch tables fit in the first two K stages");
    __shared__ int32_t perm[kMaxRankedRequests];   // request of each rank
    __shared__ int32_t order[kMaxRankedJobs];      // this XCD's work unit of each rank
    __shared__ int32_t redo;

    // Work units are jobs (group, query tile), a group being one (request, KV head), or
    // key ranges of jobs when splitting.  Workgroup L runs on XCD L % 8 (workgroups are
    // handed to the XCDs round-robin), and the jobs of group g all run on XCD g % 8: the
    // query tiles of a group read the same K/V pages, which then stay in that XCD's L2.
    // Requests are ranked by key count, longest first, and group g belongs to the
    // request of rank g / Hkv, so that every request's heads are spread over the 8 XCDs
    // (with a multiple of 8 KV heads they are whatever the order, and when the units are
    // ranked the requests are not).
    // The grid holds n_slots workgroups per XCD (no more than can run at once), each of
    // which runs a list of its XCD's units: they are ranked by key tiles, longest first,
    // and dealt to S lists in snake order (round k gives rank kS + v, or kS + S-1-v in
    // odd rounds, to list v), so that the long units start first and each list's short
    // ones balance its long ones; the lists are then placed on the CUs by their load.
    // Workgroups started by the hardware as others end would wait for a slot on their own
    // XCD; these never wait.  Every workgroup derives the
    // same orders from cu_q / cu_k in LDS; beyond kMaxRankedRequests requests or
    // kMaxRankedJobs units per XCD the batch order is kept instead.
    const int L = blockIdx.x;
    const int xcd = L % kXcds;
    const int slot = L / kXcds;
    const int tid = threadIdx.x;
    const int batch = n_groups / num_kv_heads;
    // work units per XCD: jobs, each cut into n_split key ranges when splitting
    const int n_jobs = (n_groups + kXcds - 1) / kXcds * n_qtiles * n_split;
    // cu_q and cu_k of up to kMaxRankedRequests requests are read into LDS once, by one
    // round of loads, for the orders and for every unit's bounds
    __shared__ int32_t cuq_s[kMaxRankedRequests + 1], cuk_s[kMaxRankedRequests + 1];
    const bool cu_lds = batch <= kMaxRankedRequests;
    if (cu_lds) {
        for (int j = tid; j <= batch; j += kPrefillThreads) {
            cuq_s[j] = cu_q[j];
            cuk_s[j] = cu_k[j];
        }
        __syncthreads();
    }
    // While the orders below are worked out, the workgroups of an XCD pull the q rows that
    // XCD will read into its L2, one 128-byte line per lane: with a multiple of 8 KV heads,
    // XCD x serves KV heads x, x+8, ... whatever the request order.  The loads go straight
    // to LDS, into this wave's slice of the last V stage, which nothing reads before this
    // wave's own tile loads (later, in order) overwrite it.
    if (cu_lds && num_kv_heads % kXcds == 0) {
        constexpr int kLines = G * D * 2 / 128;  // lines of one token's q rows of one KV head
        const int hpx = num_kv_heads / kXcds;    // KV heads per XCD
        const int sum_q = cuq_s[batch];
        const int64_t lines = static_cast<int64_t>(sum_q) * hpx * kLines;
        if (lines * 128 <= kQPrefetchBytes) {
            const int64_t q_bytes = static_cast<int64_t>(sum_q) * num_heads * D * 2;
            const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(q), 0, static_cast<int32_t>(min(q_bytes, static_cast<int64_t>(INT32_MAX))),
                kBufferDword3);
            const int per = n_slots * kPrefillThreads;  // lanes of the XCD
            for (int64_t l0 = 0; l0 < lines; l0 += per) {  // (uniform trip count)
                const int64_t line = l0 + slot * kPrefillThreads + tid;
                int32_t off = INT32_MIN;  // past the bound: no load
                if (line < lines) {
                    const int64_t c = line / kLines;
                    const int token = static_cast<int>(c / hpx), hkv = xcd + kXcds * static_cast<int>(c % hpx);
                    const int64_t o = (static_cast<int64_t>(token) * num_heads + hkv * G) * D * 2 + (line % kLines) * 128;
                    off = o < INT32_MAX ? static_cast<int32_t>(o) : INT32_MIN;
                }
                load_lds4(qrs, v_st3 + (kPrefillKeys / kPrefillWaves) * (tid / kWave) * D, off);
            }
        }
    }
    // key tiles of a job: -1 when its first token is past the request's queries
    // (cq, ck: the LDS copies of cu_q, cu_k, or the global arrays past kMaxRankedRequests
    // requests; each kind of call is its own loop, so no read goes through a generic pointer)
    auto job_tiles = [&](const auto* cq, const auto* ck, int req, int tok0) {
        const int q_len = cq[req + 1] - cq[req];
        if (tok0 >= q_len) return -1;
        const int k_len_req = ck[req + 1] - ck[req];
        const int k_len = kPaged ? min(k_len_req, max_blocks * BS) : k_len_req;
        const int tok_last = min(tok0 + TOK, q_len) - 1;
        const int kv_end = causal ? min(k_len, k_len_req - q_len + tok_last + 1) : k_len;
        return (kv_end > 0 && (!kPaged || num_blocks > 0)) ? (kv_end + BN - 1) / BN : 0;
    };
    // key tiles of split s of a job with `tiles` tiles: -1 when the job has no such split
    auto unit_tiles = [&](int tiles, int s) {
        if (n_split == 1 || tiles < 0) return tiles;
        const int parts = split_count(tiles, n_split, split_tiles);
        if (s >= parts) return -1;
        return parts == 1 ? tiles : (s == parts - 1 ? tiles - s * split_tiles : split_tiles);
    };
    const bool rank_jobs = n_jobs > 1 && n_jobs <= kMaxRankedJobs;
    // (with a multiple of 8 KV heads, XCD x serves heads x, x+8, ... of every request
    // whatever their order, and the job order alone makes the schedule: no request order)
    const bool rank_requests = cu_lds && batch > 1 && !(rank_jobs && num_kv_heads % kXcds == 0);
    int32_t* const klen = reinterpret_cast<int32_t*>(k_st0);  // key count of each request
    int32_t* const jobs = klen + kMaxRankedRequests;             // sort key of each unit
    int32_t* const rtiles = reinterpret_cast<int32_t*>(k_st1);   // key tiles of each rank
    if (rank_requests) {
        const int padded = (batch + 3) & ~3;  // whole 16-byte reads; -1 pads (below any count)
        for (int j = tid; j < padded; j += kPrefillThreads)
            klen[j] = j < batch ? cuk_s[j + 1] - cuk_s[j] : -1;
        lds_barrier();
        const int4* const klen4 = reinterpret_cast<const int4*>(klen);
        for (int j = tid; j < batch; j += kPrefillThreads) {
            const int kj = klen[j];
            int ahead = 0;  // requests before j in the order: longer, or as long and earlier
#pragma unroll 4
            for (int i = 0; i < padded / 4; ++i) {
                const int4 k4 = klen4[i];
                ahead += (k4.x > kj) | ((k4.x == kj) & (4 * i + 0 < j));
                ahead += (k4.y > kj) | ((k4.y == kj) & (4 * i + 1 < j));
                ahead += (k4.z > kj) | ((k4.z == kj) & (4 * i + 2 < j));
                ahead += (k4.w > kj) | ((k4.w == kj) & (4 * i + 3 < j));
            }
            perm[ahead] = j;
        }
        lds_barrier();
    }
    auto request_of = [&](int rank) { return rank_requests ? perm[rank] : rank; };
    if (rank_jobs) {
        // unit c of this XCD: job c / n_split (group (job / n_qtiles) * 8 + xcd, query
        // tile job % n_qtiles), key range c % n_split.  Its sort key packs the key tiles
        // (+1, so that -1 for "no unit" stays non-negative) above 0xFFFF - c, so that keys
        // are distinct and a larger key means "earlier": more tiles, or as many and a lower
        // index.  The rank of unit c is the number of larger keys; the table is padded
        // with zeros (below every key) to whole 16-byte reads.
        const int padded = (n_jobs + 3) & ~3;
        auto job_key = [&](int c, const auto* cq, const auto* ck) {
            int32_t key = 0;
            if (c < n_jobs) {
                const int job = c / n_split;
                const int g = (job / n_qtiles) * kXcds + xcd;
                const int tiles = g < n_groups ? job_tiles(cq, ck, request_of(g / num_kv_heads), (job % n_qtiles) * TOK) : -1;
                const int ut = unit_tiles(tiles, c % n_split);
                key = (min(ut + 1, 0x7FFE) << 16) | (0xFFFF - c);
            }
            return key;
        };
        if (cu_lds) {
            for (int c = tid; c < padded; c += kPrefillThreads) jobs[c] = job_key(c, cuq_s, cuk_s);
        } else {
            for (int c = tid; c < padded; c += kPrefillThreads) jobs[c] = job_key(c, cu_q, cu_k);
        }
        lds_barrier();
        // tpj neighbouring lanes count the larger keys of one unit, each over a share of
        // the table, and add their counts
        const int4* const jobs4 = reinterpret_cast<const int4*>(jobs);
        const int tpj = n_jobs <= kPrefillThreads / 4 ? 4 : n_jobs <= kPrefillThreads / 2 ? 2 : 1;
        const int sub = tid % tpj;
        for (int c = tid / tpj; c < n_jobs; c += kPrefillThreads / tpj) {
            const int32_t v = jobs[c];
            int ahead = 0;
#pragma unroll 4
            for (int i = sub; i < padded / 4; i += tpj) {
                const int4 u = jobs4[i];
                ahead += (u.x > v) + (u.y > v) + (u.z > v) + (u.w > v);
            }
            if (tpj > 1) ahead += __shfl_xor(ahead, 1);
            if (tpj > 2) ahead += __shfl_xor(ahead, 2);
            if (sub == 0) {
                order[ahead] = c;
                rtiles[ahead] = (v >> 16) - 1;  // -1: no unit
            }
        }
        lds_barrier();
    }
    // Placement of the lists on the CUs.  The deal above makes n_slots lists (list v: ranks
    // kS + v in even rounds k, kS + S-1-v in odd ones); which workgroup runs which list
    // decides which lists share a CU.  The hardware puts workgroup slot s of an XCD on CU
    // s mod C (C its CUs) on the first pass and slot s + C on the same CU on the second,
    // and two workgroups on one CU share its SIMDs: each runs ~1 us per key tile while both
    // are busy, ~0.75 us alone.  A CU's end is then set by its heavier list, which runs
    // alone once the lighter one is done, so the heaviest lists get CUs of their own (when
    // there are fewer than 2C slots) and each remaining CU pairs the heaviest list left with
    // the lightest (the heavier on the first-pass slot, whose waves are older and win ties
    // for the SIMD).  Only the speed depends on where a workgroup actually runs: every list
    // is run by exactly one workgroup whatever the placement.
    int list = slot;
    if (rank_jobs && cus_per_xcd > 0 && n_slots > cus_per_xcd && n_slots <= 2 * cus_per_xcd &&
        n_slots <= kMaxPlacedSlots) {
        // Every wave computes the load of each list (lane v: list v, the key tiles of its
        // units and kUnitCostTiles per unit) into a table of its own; the four waves then
        // rank a quarter of the lists each (four lanes per list, each against a quarter of
        // the table) into the shared table of lists by load rank.
        static_assert(kMaxPlacedSlots == kWave && kMaxPlacedSlots == 16 * kPrefillWaves,
                      "a list per lane; 16 lists ranked per wave");
        __shared__ __align__(16) int32_t vkeys[kPrefillWaves][kMaxPlacedSlots];
        __shared__ int32_t by_load[kMaxPlacedSlots];
        const int v = tid % kWave;
        const int wv = tid / kWave;
        int32_t* const vkey = vkeys[wv];
        int load = 0;
        if (v < n_slots) {
            const int r0 = v, r1 = 2 * n_slots - 1 - v;  // the first two rounds
            const int t0 = r0 < n_jobs ? rtiles[r0] : -1, t1 = r1 < n_jobs ? rtiles[r1] : -1;
            load = (t0 >= 0 ? t0 + kUnitCostTiles : 0) + (t1 >= 0 ? t1 + kUnitCostTiles : 0);
            for (int k = 2;; ++k) {
                const int rank = k * n_slots + (k % 2 == 0 ? v : n_slots - 1 - v);
                if (rank >= n_jobs) break;
                const int tiles = rtiles[rank];
                if (tiles >= 0) load += tiles + kUnitCostTiles;
            }
        }
        // distinct keys, a larger one meaning "heavier": more load, or as much and a lower
        // index (-1 past the lists: below all)
        vkey[v] = v < n_slots ? (min(load, (1 << 23) - 1) << 7) | (kMaxPlacedSlots - 1 - v) : -1;
        // (a wave reads its own LDS writes in order; the asm keeps the compiler from waiting
        // here for the q-row loads into the last V stage, which do not touch this table)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int list_r = 16 * wv + v / 4, sub = v % 4;
        const int32_t kr = vkey[list_r];
        const int4* const part = reinterpret_cast<const int4*>(vkey) + 4 * sub;
        int heavier = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int4 u = part[i];
            heavier += (u.x > kr) + (u.y > kr) + (u.z > kr) + (u.w > kr);
        }
        heavier += __builtin_amdgcn_update_dpp(0, heavier, 0xB1, 0xF, 0xF, false);  // lane ^ 1
        heavier += __builtin_amdgcn_update_dpp(0, heavier, 0x4E, 0xF, 0xF, false);  // lane ^ 2
        if (sub == 0 && list_r < n_slots) by_load[heavier] = list_r;
        lds_barrier();
        const int n_pairs = n_slots - cus_per_xcd;  // CUs running two workgroups of this XCD
        const int n_solo = cus_per_xcd - n_pairs;   // CUs running one
        const int load_rank = slot < n_pairs ? n_solo + slot                          // first pass, paired
                            : slot < cus_per_xcd ? slot - n_pairs                     // alone on its CU
                            : n_slots - 1 - (slot - cus_per_xcd);                     // second pass
        list = by_load[load_rank];
    }
    // (the scratch tables in the first two K stages are free once every wave is past the first
    // barrier of its first unit)

    auto run_unit = [&](int c) {
    const int job = c / n_split;
    const int group = (job / n_qtiles) * kXcds + xcd;
    // ranked: query tiles in index order; batch order: the later ones (which see more
    // keys under the causal mask) first, the key ranges of a job next to each other
    const int qtile = rank_jobs ? job % n_qtiles : n_qtiles - 1 - job % n_qtiles;
    const int split = c % n_split;
    if (group >= n_groups) return;  // uniform: grid padding
    const int hkv = group % num_kv_heads;
    const int req = __builtin_amdgcn_readfirstlane(request_of(group / num_kv_heads));  // scalar addressing
    // the request's bounds from LDS (past kMaxRankedRequests requests this unit's four
    // values are copied there first: every read of them is then an LDS read)
    int ci = req;
    if (!cu_lds) {
        if (tid == 0) {
            cuq_s[0] = cu_q[req], cuq_s[1] = cu_q[req + 1];
            cuk_s[0] = cu_k[req], cuk_s[1] = cu_k[req + 1];
        }
        __syncthreads();  // (the unit before ended with a barrier after its last read)
        ci = 0;
    }
    const int q0 = __builtin_amdgcn_readfirstlane(cuq_s[ci]);
    const int k0_req = __builtin_amdgcn_readfirstlane(cuk_s[ci]);
    const int q_len = __builtin_amdgcn_readfirstlane(cuq_s[ci + 1]) - q0;
    const int tok0 = qtile * TOK;
    if (tok0 >= q_len) return;  // uniform: tile past this request's queries
    const int k_len_req = __builtin_amdgcn_readfirstlane(cuk_s[ci + 1]) - k0_req;
    const int cached = k_len_req - q_len;                       // may be negative
    const int k_len = kPaged ? min(k_len_req, max_blocks * BS) : k_len_req;  // keys past the table: never read
    const int tok_last = min(tok0 + TOK, q_len) - 1;
    const int kv_end = causal ? min(k_len, cached + tok_last + 1) : k_len;
    const int n_tiles = (kv_end > 0 && (!kPaged || num_blocks > 0)) ? (kv_end + BN - 1) / BN : 0;
    // this unit's key tiles [t_lo, t_hi): the whole job, or one of its key ranges
    const int n_split_job = n_split == 1 ? 1 : split_count(n_tiles, n_split, split_tiles);
    if (split >= n_split_job) return;  // uniform: the job has no such key range
    const int t_lo = split * split_tiles;  // 0 when the job is not split
    const int t_hi = split == n_split_job - 1 ? n_tiles : t_lo + split_tiles;
    const int lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave index, kept in a scalar
    const int h = lane / 32;      // which 8-wide half of a 16-wide k-step this lane feeds
    const int r = lane % 32;
    // with a group size that does not divide the rows (3, 5, 6, 7) the last rows past
    // TOK whole tokens are idle: they would belong to the next workgroup's first token
    constexpr bool kAllRows = TOK * G == kPrefillRows;
    constexpr int kUsedRows = TOK * G;
    // the two rows of this lane: row block rb holds workgroup row 64w + 32rb + r
    int tok[RB], head[RB], row_limit[RB];
    bool row_ok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = kWaveRows * w + 32 * rb + r;
        tok[rb] = tok0 + row / G;
        head[rb] = hkv * G + row % G;
        row_ok[rb] = tok[rb] < q_len && (kAllRows || row < kUsedRows);
        // last key the row may see (the causal limit and the request's end)
        row_limit[rb] = min(causal ? cached + tok[rb] : k_len - 1, kv_end - 1);
    }
    const int first_row = kWaveRows * w;
    const int last_row = kAllRows ? first_row + kWaveRows - 1 : min(first_row + kWaveRows - 1, kUsedRows - 1);
    // a wave whose rows all lie past the request's queries (the last query tile of a
    // request, a decode step's single token) only stages K/V
    const bool wave_rows = first_row < kUsedRows && tok0 + first_row / G < q_len;
    const int wave_first = min(tok0 + first_row / G, q_len - 1);
    const int wave_last = min(tok0 + last_row / G, q_len - 1);
    const int wave_lo = min(causal ? cached + wave_first : k_len - 1, kv_end - 1);  // all rows see keys <= this
    const int wave_hi = wave_rows ? min(causal ? cached + wave_last : k_len - 1, kv_end - 1) : -1;
    // tiles this wave computes: [t_lo, t_end) (the keys past wave_hi are masked for all
    // its rows)
    const int t_end = max(t_lo, min(t_hi, wave_hi < 0 ? t_lo : wave_hi / BN + 1));

    // q rows of this lane, pieces 16s + 8h .. +8 of the head dim
    bf16x8_t qf[RB][KS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const uint16_t* qrow = q + (static_cast<int64_t>(q0 + tok[rb]) * num_heads + head[rb]) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok[rb]) u = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * h);
            qf[rb][s] = __builtin_bit_cast(bf16x8_t, u);
        }
    }

    f32x16_t acc[RB][DB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[rb][db][x] = 0.f;
    float m_ref[RB], lsum[RB];  // row reference (base 2, scaled; same in lanes l, l^32), this lane's part of the row sum
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_ref[rb] = -INFINITY;
        lsum[rb] = 0.f;
    }

    const int32_t* table_row = kPaged ? block_table + static_cast<int64_t>(req) * max_blocks : nullptr;
    const int64_t key_base = kPaged ? 0 : k0_req;  // first packed row of the request (contiguous)
    const int32_t row_stride = num_kv_heads * D * 2;  // bytes per slot

    // ---- loader ---------------------------------------------------------------------
    // Tiles arrive in LDS by direct loads (buffer_load ... lds): a load instruction
    // writes its 64 lanes' 16-byte pieces to 1 KB of LDS in lane order, so the loader
    // picks, for every LDS slot, which piece of global memory lands there.  Wave w loads
    // keys [8w, 8w+8) of every tile (they lie in one page: the page's address is a
    // scalar and each lane's offsets inside it never change), KPI keys per instruction,
    // K and V alike.  Rows are key-major, D elements each, and the 16-byte chunks of a
    // row are permuted (an XOR of the chunk index with a function of the key), which
    // keeps the operand reads below free of bank conflicts.  A buffer descriptor bounded
    // to the slice's valid keys makes every other lane load zeros (keys past kv_end or
    // past the unit, and the whole slice of a block id outside the pool), so nothing
    // masked can be NaN.
    constexpr int KPI = kWave * 16 / (2 * D);  // keys per load instruction: 4 (d 128), 8 (d 64)
    constexpr int NIK = SLICE / KPI;           // K (and V) load instructions per wave and tile
    // chunk permutations.  K is read 16 keys x one chunk at a time (one chunk per lane):
    // those must fall in 16 different 16-byte bank groups.  V is read transposed, 4 keys
    // x 4 chunks at a time: the keys' 64 bytes must fall in different quarters of the
    // 256-byte bank space.
    auto swz_k = [](int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); };
    auto swz_v = [](int key) { return D == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1); };
    int32_t voff_k[NIK], voff_v[NIK];
#pragma unroll
    for (int j = 0; j < NIK; ++j) {
        const int kl = KPI * j + lane / CHUNKS;  // key inside the wave's slice
        const int kt = SLICE * w + kl;           // key inside the tile
        const int p = lane % CHUNKS;             // LDS slot of the row
        voff_k[j] = kl * row_stride + 16 * (p ^ swz_k(kt));
        voff_v[j] = kl * row_stride + 16 * (p ^ swz_v(kt));
    }
    const int64_t head_off = static_cast<int64_t>(hkv) * D * 2;

    // Block ids of the pages of four tiles at a time come from one vector load (lane i
    // holds page i of them), issued four tiles ahead of their use (scalar loads would
    // hold up the LDS waits, which share their counter); a tile's ids are moved to scalar
    // registers when its loads are prepared.
    const __amdgpu_buffer_rsrc_t table_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(kPaged ? table_row : cu_k), 0, kPaged ? max_blocks * 4 : 0,
        kBufferDword3);
    auto load_idq = [&](int t0) -> uint32_t {  // ids of tiles [t0, t0+4); zero past the table
        if constexpr (!kPaged) {
            return 0u;
        } else {
            const int i = lane < 4 * PAGES ? lane : 0;  // (other lanes: a copy of lane 0's word)
            return __builtin_amdgcn_raw_buffer_load_b32(table_rsrc, (t0 * PAGES + i) * 4, 0, 0);
        }
    };
    struct TileIds {
        uint32_t bits;  // bit i: page i is past kv_end or holds a block id inside the pool
        int32_t wave;   // block id of this wave's slice
    };
    // ids of tile t, the k-th tile of the four in idq
    auto scalar_ids = [&](int t, uint32_t idq, int k) {
        TileIds res{(1u << PAGES) - 1, 0};
        if constexpr (kPaged) {
            res.bits = 0;
#pragma unroll
            for (int i = 0; i < PAGES; ++i) {
                const int32_t id = __builtin_amdgcn_readlane(static_cast<int32_t>(idq), k * PAGES + i);
                const bool past = t * BN + i * PBS >= kv_end;
                res.bits |= (past || static_cast<uint32_t>(id) < static_cast<uint32_t>(num_blocks) ? 1u : 0u) << i;
                if ((SLICE * w) / PBS == i) res.wave = id;
            }
        }
        return res;
    };
    // the loads of this wave's slice of tile t: their two descriptors (K, V), then the
    // 2 NIK instructions one by one (issue), or all of them (load_tile)
    struct TileRsrc {
        __amdgpu_buffer_rsrc_t k, v;
    };
    // Constants of the descriptors: the slice's offset inside a page (tiles are whole
    // pages or whole multiples of them) with the head, as base pointers; keys past
    // unit_end (the unit's last tile or kv_end) load zeros.
    const int unit_end = min(kv_end, t_hi * BN);
    const int64_t slice_off = kPaged ? static_cast<int64_t>((SLICE * w) % PBS) * row_stride + head_off
                                     : (key_base + SLICE * w) * row_stride + head_off;
    const char* const k_slice = k_cache + slice_off;
    const char* const v_slice = v_cache + slice_off;
    const uint32_t step_bytes = (kPaged ? PBS : BN) * static_cast<uint32_t>(row_stride);  // per block id / tile
    auto tile_rsrc = [&](int t, int32_t id) {
        int32_t bytes = min(max(unit_end - (t * BN + SLICE * w), 0), SLICE) * row_stride;
        uint32_t index = static_cast<uint32_t>(t);
        if constexpr (kPaged) {
            const bool in_pool = static_cast<uint32_t>(id) < static_cast<uint32_t>(num_blocks);
            index = in_pool ? static_cast<uint32_t>(id) : 0u;
            bytes = in_pool ? bytes : 0;
        }
        // (readfirstlane: values the compiler would form on the vector unit would turn
        // each load into a loop over lanes)
        bytes = __builtin_amdgcn_readfirstlane(bytes);
        index = __builtin_amdgcn_readfirstlane(index);
        const uint64_t off = static_cast<uint64_t>(index) * step_bytes;
        return TileRsrc{__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(k_slice + off), 0, bytes, kBufferDword3),
                        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(v_slice + off), 0, bytes, kBufferDword3)};
    };
    auto issue = [&](auto st, const TileRsrc& rs, int j) {
        if (j < NIK)
            load_lds16(rs.k, k_of(st) + (SLICE * w + KPI * j) * D, voff_k[j]);
        else
            load_lds16(rs.v, v_of(st) + (SLICE * w + KPI * (j - NIK)) * D, voff_v[j - NIK]);
    };
    auto load_tile = [&](auto st, int t, int32_t id) {
        const TileRsrc rs = tile_rsrc(t, id);
#pragma unroll
        for (int j = 0; j < 2 * NIK; ++j) issue(st, rs, j);
    };

    // ---- operand reads ----------------------------------------------------------------
    // K (A operand of S^T = K Q^T): key r of the tile, dims 16ks + 8h .. +8, one 16-byte
    // read per k-step.
    int32_t k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = r * D + 8 * ((2 * ks + h) ^ swz_k(r));
    auto read_k = [&](auto st, int ks) {
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(k_of(st) + k_rd[ks]));
    };
    // V^T (A operand of O^T += V^T P^T): for dims 32db + r, the 8 keys that the P^T
    // operand holds at contraction positions 8h .. 8h+7 of k-step ks, which are keys
    // 16ks + 4h + e and 16ks + 8 + 4h + e (e < 4; the order in which the S^T accumulators
    // hold a lane's keys).  Two transposing reads (ds_read_b64_tr_b16) of 4 keys each: in
    // every 16-lane group, lane 4e + q supplies the address of 4 consecutive dims of key e,
    // and lane j receives dim j%4 of the 4 keys supplied by lanes 4e + (j%16)/4.  Lane
    // s = 16g + 4e + q therefore points at key 4(g/2) + e (+8, +16ks), dims
    // 32db + 16(g%2) + 4q.
    int32_t v_rd[DB];
    {
        const int g = lane / 16, e = (lane / 4) % 4, q4 = lane % 4;
        const int key = 4 * (g / 2) + e;  // swz_v depends on key bits that 16ks and 8 keep
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int chunk = 4 * db + 2 * (g % 2) + q4 / 2;
            v_rd[db] = key * D + 8 * (chunk ^ swz_v(key)) + 4 * (q4 % 2);
        }
    }
    auto read_v = [&](auto st, int db, int ks) {
        const uint16_t* p = v_of(st) + v_rd[db] + 16 * ks * D;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(to_lds_v4(p));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(to_lds_v4(p + 8 * D));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // S^T of a tile: s[rb] accumulates keys 8(x/4) + 4h + x%4 of the tile for row block rb
    auto zero_s = [&](f32x16_t (&s)[RB]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int x = 0; x < 16; ++x) s[rb][x] = 0.f;
    };
    auto qk = [&](auto st, f32x16_t (&s)[RB]) {
        zero_s(s);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t a = read_k(st, ks);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][ks], s[rb], 0, 0, 0);
        }
    };
    // References.  Each row's reference is the maximum of its scores in the unit's first
    // tile (0 for a row with no visible key there), and the weights exp2(s - reference)
    // are never rescaled, so O is touched by nothing but the matrix products.  A later
    // score far above the reference shows as a tile's weight sum above 2^64 (or not
    // finite); the workgroup then flags the unit and computes it again, first the exact
    // row maxima (a pass over the scores alone), then the attention against them.
    // A tile's 16 weights per lane and row block come in pairs: pair pr is elements e, e+1
    // of the P^T operand pb[rb][hf] (hf = pr / 4RB, rb = (pr % 4RB) / 4, e = 2 (pr % 4)),
    // from the accumulators 8hf + e, +1 of the scores of row block rb.  Their row sums go
    // to two independent partial sums per row block.
    auto weight_pair = [&](const f32x16_t (&sc)[RB], const float (&mu)[RB], int pr, bf16x8_t (&pb)[RB][2]) {
        const int hf = pr / (4 * RB), rb = (pr % (4 * RB)) / 4, e = 2 * (pr % 4);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[rb][8 * hf + e], qscale, -mu[rb]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[rb][8 * hf + e + 1], qscale, -mu[rb]));
        const bf16x2_t pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
        pb[rb][hf][e] = pp[0];
        pb[rb][hf][e + 1] = pp[1];
    };
    auto pair_sum = [&](const bf16x8_t (&pb)[RB][2], int pr, float (&part)[RB][2]) {
        const int hf = pr / (4 * RB), rb = (pr % (4 * RB)) / 4, e = 2 * (pr % 4);
        const bf16x2_t pp = {pb[rb][hf][e], pb[rb][hf][e + 1]};
        part[rb][pr % 2] = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, part[rb][pr % 2], false);
    };
    // A step in two phases (two waves per SIMD): first its 16 products back to back (tile
    // t+1's scores, then tile t's P V) at raised priority, then tile t+1's weights and row
    // sums at normal priority.  The wave in its products keeps the matrix core busy while
    // the other wave of the SIMD issues its vector work; the matrix core, which the two
    // share, makes them take turns.  (Weights spread between the products of the same
    // wave, or no priority, measured slower.)
    constexpr int kAhead = 4;  // operand reads in flight ahead of their products
    // The products: tile t+1's scores (K from stage sk) and tile t's P V (V^T from stage
    // sv).  The loads of tile t+3 (2 NIK instructions) are issued between the score
    // products, the first kAhead V^T reads during the last score k-steps (so the first P V
    // product finds its operand in), and mid() (scalar work of the loader) next to the
    // second P V product; sched_barrier(0) fences keep that order.
    auto products = [&](auto sk, auto sv, f32x16_t (&sn)[RB], const bf16x8_t (&pb)[RB][2], auto lst,
                        const TileRsrc& rs, auto&& mid) {
        constexpr int NO = 2 * DB;
        zero_s(sn);
        bf16x8_t a[KS];
        bf16x8_t va[NO];
#pragma unroll
        for (int ks = 0; ks < kAhead; ++ks) a[ks] = read_k(sk, ks);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + kAhead < KS) a[ks + kAhead] = read_k(sk, ks + kAhead);
            else va[ks + kAhead - KS] = read_v(sv, (ks + kAhead - KS) % DB, (ks + kAhead - KS) / DB);
#pragma unroll
            for (int j = 2 * NIK * ks / KS; j < 2 * NIK * (ks + 1) / KS; ++j) issue(lst, rs, j);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                sn[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[rb][ks], sn[rb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < NO; ++i) {
            const int ks = i / DB, db = i % DB;
            if (i + kAhead < NO) va[i + kAhead] = read_v(sv, (i + kAhead) % DB, (i + kAhead) / DB);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[rb][ks], acc[rb][db], 0, 0, 0);
            if (i == 1) mid();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // The weights of a tile (scores s) into pb and their row sums into lsum.  A tile whose
    // sums are not finite or above 2^64 (a score far above its row's reference) flags the
    // unit to be computed again against exact row maxima.
    auto weights = [&](const f32x16_t (&s)[RB], bf16x8_t (&pb)[RB][2]) {
        float part[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) part[rb][0] = part[rb][1] = 0.f;
#pragma unroll
        for (int pr = 0; pr < NP; ++pr) weight_pair(s, m_ref, pr, pb);
#pragma unroll
        for (int pr = 0; pr < NP; ++pr) pair_sum(pb, pr, part);
        bool over = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float ps = part[rb][0] + part[rb][1];
            lsum[rb] += ps;
            over = over || !(ps <= kFastSumLimit);
        }
        if (over) redo = 1;
    };

    // masking of tile t: keys past a row's limit, keys of an unassigned block (none
    // in most tiles: the caller tests need_mask first)
    // (tile t has a key past wave_lo iff t >= t_mask)
    const int t_mask = (wave_lo + 1) / BN;  // wave_lo >= -1
    auto need_mask = [&](int t, uint32_t page_ok) {
        return page_ok != (1u << PAGES) - 1 || t >= t_mask;
    };
    auto mask = [&](int t, f32x16_t (&s)[RB], uint32_t page_ok) {
        const int j0 = t * BN;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int lim = row_limit[rb] - j0 - 4 * h;  // keys 8(x/4) + x%4 <= lim are visible
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int key = 8 * (x / 4) + (x % 4);
                s[rb][x] = key <= lim ? s[rb][x] : -INFINITY;
            }
        }
        if (page_ok != (1u << PAGES) - 1) {
            // accumulator x holds key 8(x/4) + 4h + x%4, in page (8(x/4)) / PBS for both lane
            // halves: a compile-time index
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int page = (8 * (x / 4)) / PBS;
                    s[rb][x] = (page_ok >> page) & 1u ? s[rb][x] : -INFINITY;
                }
        }
    };
    // row maxima of a tile's scores (scaled to base 2; lanes l and l^32 agree)
    auto tile_max = [&](const f32x16_t (&s)[RB], float (&mx)[RB]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float v = -INFINITY;
#pragma unroll
            for (int x = 0; x < 16; ++x) v = fmaxf(v, s[rb][x]);
            mx[rb] = fmaxf(v, __shfl_xor(v, 32)) * qscale;  // qscale > 0: the max scales with it
        }
    };
    // O stays in vector registers, where the products accumulate it: nothing else touches
    // it until the end
    auto pin_acc = [&]() {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(acc[rb][db]));
    };

    // ---- the key loop ---------------------------------------------------------------
    // One pass over the unit's tiles: the attention (MAX_ONLY false), or the row maxima
    // of the scores alone into m_ref (MAX_ONLY true).  Four LDS stages: at step t the
    // wave computes tile t+1's scores (stage of t+1) and tile t's P V (stage of t), while
    // the loads of tiles t+2 and t+3 are in flight, so a load has two steps to land.
    // Step t starts by waiting for its own loads of tile t+1 (all but the last step's
    // vector-memory instructions: 2 NIK tile loads, and one block-id load on the first
    // step of a loop trip when paged) and a barrier, after which tile t+1 is complete in
    // LDS and every wave is done with tile t-1's stage, into which tile t+3 is then
    // loaded.  The stage of a tile is fixed by its position in the unit, so the loop is
    // unrolled four times and every LDS address is static.  Both waves run every step
    // (the loads and barriers are shared); a wave computes only tiles before its t_end.
    const int n = t_hi - t_lo;
    auto key_pass = [&](auto max_only, bool set_refs) {
        constexpr bool MAX_ONLY = decltype(max_only)::value;
        if (n <= 0) return;
        uint32_t okq;      // page bits of tiles t .. t+4 at bits 0, 2, 4, 6, 8
        uint32_t idq_cur;  // block ids of tiles [t0+4, t0+8), t0 the first tile of the loop trip
        uint32_t idq_next; // those of [t0+8, t0+12), loaded during the trip
        TileRsrc rs3;      // descriptors of the loads of tile t+3 at step t
        f32x16_t sa[RB], sb[RB];
        bf16x8_t pbuf[RB][2];  // weights of the tile whose P V comes next
        // scores are read by vector instructions: keep them in vector registers
        auto pin_s = [&](f32x16_t (&s)[RB]) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) asm volatile("" : "+v"(s[rb]));
        };
        {
            const uint32_t q0 = load_idq(t_lo);
            idq_cur = load_idq(t_lo + 4);
            __syncthreads();  // LDS of the job orders or of the pass before: no longer read
            const TileIds a0 = scalar_ids(t_lo, q0, 0), a1 = scalar_ids(t_lo + 1, q0, 1),
                          a2 = scalar_ids(t_lo + 2, q0, 2), a3 = scalar_ids(t_lo + 3, q0, 3);
            load_tile(Stage<0>{}, t_lo, a0.wave);
            load_tile(Stage<1>{}, t_lo + 1, a1.wave);
            load_tile(Stage<2>{}, t_lo + 2, a2.wave);
            rs3 = tile_rsrc(t_lo + 3, a3.wave);
            okq = a0.bits | (a1.bits << 2) | (a2.bits << 4) | (a3.bits << 6);
            wait_loads_and_barrier<4 * NIK>();  // tile t_lo in LDS (the later loads may fly)
            if (t_lo < t_end) {
                qk(Stage<0>{}, sa);
                pin_s(sa);
                if (!MAX_ONLY && set_refs) {
                    if (need_mask(t_lo, okq & 3u)) mask(t_lo, sa, okq & 3u);
                    float mx[RB];
                    tile_max(sa, mx);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) m_ref[rb] = mx[rb] == -INFINITY ? 0.f : mx[rb];
                }
            }
            if (!MAX_ONLY && set_refs && t_lo >= t_end) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) m_ref[rb] = 0.f;
            }
            if constexpr (!MAX_ONLY) {
                // the weights of tile t_lo, for the first step's P V
                if (t_lo < t_end) {
                    if (!set_refs && need_mask(t_lo, okq & 3u)) mask(t_lo, sa, okq & 3u);
                    weights(sa, pbuf);
                }
            }
        }
        // Step t (the ST-th of its loop trip): tile t in stage ST; tile t+1's scores go to
        // sn.  The attention pass runs the products (tile t+1's scores, tile t's P V with
        // the weights pbuf made the step before), then tile t+1's weights into pbuf; the
        // max-only pass takes the maxima of tile t's scores (sc) and computes tile t+1's.
        // The loads of tile t+3 (descriptors made at step t-1) are issued between the
        // score products, the descriptors of tile t+4 made between the P V products; the
        // first step of a trip loads the block ids of the trip after next.  A step issues
        // 2 NIK loads, the first of a trip one more (after its tile loads), which fixes how
        // many of them the next step's wait leaves in flight.
        auto step = [&](auto st, int t, f32x16_t (&sc)[RB], f32x16_t (&sn)[RB]) {
            constexpr int ST = decltype(st)::value;
            wait_loads_and_barrier<2 * NIK + (ST == 1 && kPaged ? 1 : 0)>();
            const TileRsrc rs = rs3;
            auto next_desc = [&]() {
                const TileIds ti = scalar_ids(t + 4, idq_cur, ST);
                rs3 = tile_rsrc(t + 4, ti.wave);
                okq |= ti.bits << 8;
            };
            constexpr auto lst = Stage<(ST + 3) % 4>{};
            if (MAX_ONLY || !(t < t_end)) {
#pragma unroll
                for (int j = 0; j < 2 * NIK; ++j) issue(lst, rs, j);
                if constexpr (ST == 0) idq_next = load_idq(t + 8);
            }
            if (t < t_end) {
                if (MAX_ONLY && need_mask(t, okq & 3u)) mask(t, sc, okq & 3u);
                if constexpr (MAX_ONLY) {
                    float mx[RB];
                    tile_max(sc, mx);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) m_ref[rb] = fmaxf(m_ref[rb], mx[rb]);
                    qk(Stage<(ST + 1) % 4>{}, sn);
                    next_desc();
                } else {
                    // tile t's weights were made at the end of the step before (or the prologue)
                    __builtin_amdgcn_s_setprio(1);
                    products(Stage<(ST + 1) % 4>{}, Stage<ST>{}, sn, pbuf, lst, rs, next_desc);
                    if constexpr (ST == 0) idq_next = load_idq(t + 8);
                    __builtin_amdgcn_s_setprio(0);
                    pin_acc();
                    if (t + 1 < t_end) {
                        const uint32_t ok1 = (okq >> 2) & 3u;  // page bits of tile t+1
                        if (need_mask(t + 1, ok1)) mask(t + 1, sn, ok1);
                        weights(sn, pbuf);
                    }
                }
                // (placed after the products, so that it does not split the stretch above)
                pin_s(sn);
            } else {
                next_desc();
            }
            okq >>= 2;
        };
        int t = t_lo;
        for (; t + 4 <= t_hi; t += 4) {
            step(Stage<0>{}, t, sa, sb);
            step(Stage<1>{}, t + 1, sb, sa);
            step(Stage<2>{}, t + 2, sa, sb);
            step(Stage<3>{}, t + 3, sb, sa);
            idq_cur = idq_next;
        }
        if (t < t_hi) step(Stage<0>{}, t, sa, sb);
        if (t + 1 < t_hi) step(Stage<1>{}, t + 1, sb, sa);
        if (t + 2 < t_hi) step(Stage<2>{}, t + 2, sa, sb);
        // the loads past the unit land before the stages are used again (or the wave ends)
        wait_loads_and_barrier<0>();
    };
    if (tid == 0) redo = 0;  // (seen by every wave after the pass's first barrier)
    pin_acc();
    key_pass(std::false_type{}, true);
    __syncthreads();  // every wave's flag is in
    const bool again = redo != 0;  // uniform: the same LDS word for the whole workgroup
    __syncthreads();  // every wave has read it (the next unit clears it)
    if (again) {
        // exact row maxima first, then the attention against them (no weight exceeds 1)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) m_ref[rb] = -INFINITY;
        key_pass(std::true_type{}, false);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m_ref[rb] = m_ref[rb] == -INFINITY ? 0.f : m_ref[rb];
            lsum[rb] = 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) acc[rb][db][x] = 0.f;
        }
        pin_acc();
        key_pass(std::false_type{}, false);
    }

    // normalise and store: lane holds d = 32db + 8i + 4h + jj of its rows
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float lt = lsum[rb] + __shfl_xor(lsum[rb], 32);
        const int row = kWaveRows * w + 32 * rb + r;
        if (kSplit && n_split_job > 1) {
            // one key range of a split job: the unnormalised O, the reference m and l of
            // each row go to the workspace, for prefill_merge_kernel
            if (!row_ok[rb]) continue;
            const int64_t unit =
                ((static_cast<int64_t>(req) * num_kv_heads + hkv) * n_qtiles + qtile) * n_split + split;
            float* prow = part_o + (unit * kPrefillRows + row) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4)
                    *reinterpret_cast<float4*>(prow + 32 * db + 8 * i4 + 4 * h) =
                        make_float4(acc[rb][db][4 * i4], acc[rb][db][4 * i4 + 1], acc[rb][db][4 * i4 + 2],
                                    acc[rb][db][4 * i4 + 3]);
            if (h == 0) part_ml[unit * kPrefillRows + row] = make_float2(lt > 0.f ? m_ref[rb] : -INFINITY, lt);
            continue;
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        // The 32 rows of the block go through LDS, so that the stores write whole 16-byte
        // pieces of a row, eight lanes per 128-byte line (a lane holds 8-byte pieces of 16
        // rows' lines otherwise, and those partial writes held the end of a unit up by
        // ~2 us).  Each wave uses its own K stage (every wave is past the key pass, whose
        // last barrier ended all reads of the stages, and the next unit loads none before
        // its first barrier); a wave reads its own LDS writes in order.  16-byte piece c
        // of row x sits at position c ^ (x mod CH) of the row, which spreads both the
        // writes and the row-wise reads over the banks.
        constexpr int CH = D / 8;             // 16-byte pieces per row
        constexpr int RPI = kWave / CH;       // rows per read instruction
        static_assert(kPrefillWaves <= kPrefillStages && 32 * D <= TILE, "a K stage holds a wave's block");
        uint16_t* const ost = w == 0 ? k_st0 : w == 1 ? k_st1 : w == 2 ? k_st2 : k_st3;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                uint32_t lo = static_cast<uint32_t>(to_bf16_bits(acc[rb][db][4 * i4 + 0] * inv)) |
                              (static_cast<uint32_t>(to_bf16_bits(acc[rb][db][4 * i4 + 1] * inv)) << 16);
                uint32_t hi = static_cast<uint32_t>(to_bf16_bits(acc[rb][db][4 * i4 + 2] * inv)) |
                              (static_cast<uint32_t>(to_bf16_bits(acc[rb][db][4 * i4 + 3] * inv)) << 16);
                const int c = 4 * db + i4;  // piece of d = 32db + 8i4 .. +8; half h of it
                *reinterpret_cast<uint2*>(ost + r * D + 8 * (c ^ (r % CH)) + 4 * h) = make_uint2(lo, hi);
            }
#pragma unroll
        for (int kk = 0; kk < 32 / RPI; ++kk) {
            const int x = RPI * kk + lane / CH, c = lane % CH;  // row x of the block, piece c
            const uint4 v = *reinterpret_cast<const uint4*>(ost + x * D + 8 * (c ^ (x % CH)));
            const int row = kWaveRows * w + 32 * rb + x;
            const int tok_x = tok0 + row / G;
            if (tok_x < q_len && (kAllRows || row < kUsedRows))
                *reinterpret_cast<uint4*>(out + (static_cast<int64_t>(q0 + tok_x) * num_heads + hkv * G + row % G) * D +
                                          8 * c) = v;
        }
    }
    };  // run_unit

    // this workgroup's units: those of its list, dealt in snake order from the XCD's ranking
    for (int k = 0;; ++k) {
        const int rank = k * n_slots + (k % 2 == 0 ? list : n_slots - 1 - list);
        if (rank >= n_jobs) break;  // (the last round: no later one)
        run_unit(rank_jobs ? order[rank] : rank);
    }
    // a workgroup whose units all turned out empty still has its q-row loads into LDS in
    // flight: they land before the wave ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace pa
