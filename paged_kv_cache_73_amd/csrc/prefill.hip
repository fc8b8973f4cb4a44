// Varlen (packed) paged prefill on the matrix cores.
//
// What it computes ("从零开始写Qwen3（六）PagedAttention", fast-attn 库的使用: the varlen call
// with a block table; "Sayfalı dikkat", Değişken uzunluklu yol): request i owns query
// rows [cu_q[i], cu_q[i+1]) of the packed q and k_len = cu_k[i+1] - cu_k[i] keys, read
// through block_table row i ("Paged attention 与 online softmax" §11.1).  With
// c = k_len - q_len cached tokens, query row t sees keys j <= c + t when causal.
//
// How (gfx950, bf16 in, fp32 accumulate):
// * One workgroup = 4 waves = 128 "rows" of one request and one KV head, a row being a
//   (token, query head) pair: the G query heads sharing the KV head are packed next to
//   each other, so every K/V tile read serves all of them.
// * The keys are walked in tiles of 64 (a whole number of pages), FlashAttention-style
//   ("结合nanovllm的FlashAttention和PagedAttention主要原理概述" 题目3): each tile is
//   gathered page by page through the block table into LDS, scores are formed, folded
//   into the running (m, l, O) with the §11.2 rule, and O is normalised once at the end.
// * Transposed products keep every query row inside one lane: S^T = K Q^T with
//   v_mfma_f32_32x32x16_bf16 (A = a K tile row per lane, B = the lane's q row), so lane
//   l holds 16 scores of query row l%32 (the other 16 of the 32-key block sit in lane
//   l^32).  The softmax is therefore lane-local apart from one exchange for the row max.
//   O^T += V^T P^T then takes P straight from the S^T accumulators (the key order inside
//   a 16-key step is permuted identically on both operands) and V^T from LDS, where the
//   loader stores V transposed, each 16-key group in that same permuted order so that
//   one operand is 16 contiguous bytes.
// * Each wave stages a 16-key slice of every tile: one page, whose address is a scalar.
//   The next tile's K/V are loaded into registers while the current tile is computed.
// * Masking selects: keys past the request, beyond the causal limit or in a block whose
//   id is outside [0, num_blocks) are set to -inf before the exponent; their K/V are
//   loaded as zeros (never from the pool), so no NaN can enter the products.
// * BS = 0 instantiates the same kernel for contiguous K/V (the varlen call without a
//   block table, "从零开始写Qwen3（六）" fast-attn 库的使用): request i's keys are rows
//   [cu_k[i], cu_k[i+1]) of packed [sum_k][Hkv][d] arrays, and only the addressing of
//   the loader differs.

#include <algorithm>
#include <atomic>

#include "common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

// Raise the wave's priority while it issues matrix products (1) or not (0).
#ifndef PA_PREFILL_SETPRIO
#define PA_PREFILL_SETPRIO 1
#endif
// MFMA operands read from LDS ahead of the product that uses them.
#ifndef PA_PREFILL_LDS_AHEAD
#define PA_PREFILL_LDS_AHEAD 4
#endif
// Padding (elements) of a V^T row in LDS.
#ifndef PA_PREFILL_VT_PAD
#define PA_PREFILL_VT_PAD 4
#endif

constexpr int kPrefillRows = 128;   // rows per workgroup (4 waves x 32)
constexpr int kPrefillKeys = 64;    // keys per tile
constexpr int kPrefillThreads = 256;
constexpr int kXcds = 8;            // accelerator complex dies of an MI355X
constexpr float kRescaleSlack = 8.f; // weights stay below 2^8 between rescales
constexpr int kMaxRankedRequests = 256;  // requests ordered by key count in-kernel
// Jobs per XCD ordered by key tiles in-kernel.  Ranking costs O(jobs^2) LDS compares per
// workgroup and separates the query tiles of a group (which then stop sharing K/V pages
// in L2); past a few jobs per workgroup slot the batch order, which keeps a group's tiles
// together, measured faster.
constexpr int kMaxRankedJobs = 384;

// Instruction order for a run of N products whose operands come from LDS: AHEAD reads
// first, then each product followed by the next read, so that AHEAD reads stay in
// flight (the scheduler otherwise moves every read next to its product).
// Key ranges of a job of `tiles` key tiles when jobs are cut into ranges of split_tiles
// tiles, at most n_split of them (the last one takes the rest).
__host__ __device__ inline int split_count(int tiles, int n_split, int split_tiles) {
    if (n_split <= 1 || tiles <= split_tiles) return 1;
    const int parts = (tiles + split_tiles - 1) / split_tiles;
    return parts < n_split ? parts : n_split;
}

template <int N, int AHEAD>
__device__ __forceinline__ void pipeline_order() {
    constexpr int kLdsRead = 0x100, kMfma = 0x008;
    __builtin_amdgcn_sched_group_barrier(kLdsRead, AHEAD, 0);
#pragma unroll
    for (int o = 0; o < N; ++o) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
        if (o + AHEAD < N) __builtin_amdgcn_sched_group_barrier(kLdsRead, 1, 0);
    }
}

// BS = 0: contiguous K/V.  kSplit: jobs may be cut into key ranges (n_split, split_tiles);
// without it those arguments are ignored and the kernel is the plain one.
template <int D, int G, int BS, bool kSplit>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    const uint16_t* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ block_table,
    uint16_t* __restrict__ out, int32_t num_heads, int32_t num_kv_heads, int32_t num_blocks,
    int32_t max_blocks, float qscale, int32_t causal, int32_t n_qtiles, int32_t n_groups,
    int32_t n_split_arg, int32_t split_tiles_arg, float* __restrict__ part_o,
    float2* __restrict__ part_ml) {
    const int n_split = kSplit ? n_split_arg : 1;
    const int split_tiles = kSplit ? split_tiles_arg : 0;
    constexpr int BN = kPrefillKeys;
    constexpr bool kPaged = BS > 0;
    constexpr int PBS = kPaged ? BS : BN;        // keys per page (one page per tile when contiguous)
    constexpr int TOK = kPrefillRows / G;       // tokens per workgroup
    constexpr int KS = D / 16;                  // MFMA k-steps over the head dim
    constexpr int DB = D / 32;                  // 32-wide blocks of the head dim in O^T
    constexpr int PITCH = D + 8;                // LDS row pitch (elements); the pad spreads banks
    constexpr int CHUNKS = D / 8;               // 16-byte pieces per K/V row
    constexpr int WAVE_KEYS = BN / 4;           // keys of a tile staged by each wave
    constexpr int KPT = WAVE_KEYS * CHUNKS / kWave;  // keys per loader thread: 4 (d 128), 2 (d 64)
    constexpr int GPW = kWave / CHUNKS;         // key groups per wave
    static_assert(KPT == 2 || KPT == 4, "loader split");
    static_assert(PBS % WAVE_KEYS == 0, "a wave's keys lie in one page");

    // V is stored transposed (V^T[d][key]) so that an O^T operand (8 keys of one dim) is
    // two 8-byte reads.  Pitch BN + 4: 8-byte aligned rows; the reads of 16 consecutive
    // rows then cover all banks once, the loader's writes conflict 2-way at most.
    constexpr int PITCH_T = BN + PA_PREFILL_VT_PAD;
    constexpr int LDS_AHEAD = PA_PREFILL_LDS_AHEAD;  // MFMA operands read ahead of use
    // K/V tiles are double-buffered: the next tile is staged while this one is read
    __shared__ __align__(16) uint16_t k_lds_all[2][BN * PITCH];
    __shared__ __align__(16) uint16_t v_lds_all[2][D * PITCH_T];
    static_assert(2 * kMaxRankedRequests <= BN * PITCH / 2 && kMaxRankedJobs <= BN * PITCH / 2,
                  "the ranking tables fit in one K tile buffer each");

    // Work items are jobs (group, query tile), a group being one (request, KV head).
    // Workgroup L runs on XCD L % 8 (workgroups are handed to the XCDs round-robin), and
    // the jobs of group g all run on XCD g % 8: the query tiles of a group read the same
    // K/V pages, which then stay in that XCD's L2.  Requests are ranked by key count,
    // longest first, and group g belongs to the request of rank g / Hkv, so that every
    // request's heads are spread over the 8 XCDs.  Within an XCD the jobs start in order
    // of decreasing key-tile count (longest-processing-time first): workgroup slot s of
    // the XCD takes the job of rank s, and the short jobs fill the gaps at the end.
    // Every workgroup derives the same orders from cu_q / cu_k in LDS (the K tile
    // buffers, overwritten only after a barrier); beyond kMaxRankedRequests requests or
    // kMaxRankedJobs jobs per XCD the batch order is kept instead.
    const int L = blockIdx.x;
    const int xcd = L % kXcds;
    const int slot = L / kXcds;
    const int tid = threadIdx.x;
    const int batch = n_groups / num_kv_heads;
    // work units per XCD: jobs, each cut into n_split key ranges when splitting
    const int n_jobs = (n_groups + kXcds - 1) / kXcds * n_qtiles * n_split;
    // key tiles of a job: -1 when its first token is past the request's queries
    auto job_tiles = [&](int req, int tok0) {
        const int q_len = cu_q[req + 1] - cu_q[req];
        if (tok0 >= q_len) return -1;
        const int k_len_req = cu_k[req + 1] - cu_k[req];
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
    const bool rank_requests = batch > 1 && batch <= kMaxRankedRequests;
    const bool rank_jobs = n_jobs > 1 && n_jobs <= kMaxRankedJobs;
    int32_t* const perm = reinterpret_cast<int32_t*>(k_lds_all[0]);  // request of each rank
    int32_t* const klen = perm + kMaxRankedRequests;                 // key count of each request
    int32_t* const jobs = reinterpret_cast<int32_t*>(k_lds_all[1]);  // key tiles of each job
    __shared__ int32_t found;
    if (rank_requests) {
        const int padded = (batch + 3) & ~3;  // whole 16-byte reads; -1 pads (below any count)
        for (int j = tid; j < padded; j += kPrefillThreads)
            klen[j] = j < batch ? cu_k[j + 1] - cu_k[j] : -1;
        __syncthreads();
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
        __syncthreads();
    }
    auto request_of = [&](int rank) { return rank_requests ? perm[rank] : rank; };
    int group, qtile, split;
    if (rank_jobs) {
        // job c of this XCD: group (c / n_qtiles) * 8 + xcd, query tile c % n_qtiles.  Its
        // sort key packs the key tiles (+1, so that -1 for "no job" stays non-negative)
        // above 0xFFFF - c, so that keys are distinct and a larger key means "earlier":
        // more tiles, or as many and a lower index.  The rank of job c is the number of
        // larger keys; the table is padded with zeros (below every key) to whole 16-byte
        // reads.
        const int padded = (n_jobs + 3) & ~3;
        for (int c = tid; c < padded; c += kPrefillThreads) {
            int32_t key = 0;
            if (c < n_jobs) {
                const int job = c / n_split;
                const int g = (job / n_qtiles) * kXcds + xcd;
                const int tiles = g < n_groups ? job_tiles(request_of(g / num_kv_heads), (job % n_qtiles) * TOK) : -1;
                const int ut = unit_tiles(tiles, c % n_split);
                key = (min(ut + 1, 0x7FFE) << 16) | (0xFFFF - c);
            }
            jobs[c] = key;
        }
        __syncthreads();
        const int4* const jobs4 = reinterpret_cast<const int4*>(jobs);
        for (int c = tid; c < n_jobs; c += kPrefillThreads) {
            const int32_t v = jobs[c];
            int ahead = 0;
#pragma unroll 4
            for (int i = 0; i < padded / 4; ++i) {
                const int4 u = jobs4[i];
                ahead += (u.x > v) + (u.y > v) + (u.z > v) + (u.w > v);
            }
            if (ahead == slot) found = c;
        }
        __syncthreads();
        const int c = __builtin_amdgcn_readfirstlane(found);
        const int job = c / n_split;
        group = (job / n_qtiles) * kXcds + xcd;
        qtile = job % n_qtiles;
        split = c % n_split;
    } else {
        // the groups of the XCD in turn, the query tiles of a group back to back, the
        // later ones (which see more keys under the causal mask) first, the key ranges
        // of a job next to each other
        const int job = slot / n_split;
        group = (job / n_qtiles) * kXcds + xcd;
        qtile = n_qtiles - 1 - job % n_qtiles;
        split = slot % n_split;
    }
    if (group >= n_groups) return;  // uniform: grid padding
    const int hkv = group % num_kv_heads;
    const int req = __builtin_amdgcn_readfirstlane(request_of(group / num_kv_heads));  // scalar addressing
    const int q0 = cu_q[req];
    const int q_len = cu_q[req + 1] - q0;
    const int tok0 = qtile * TOK;
    if (tok0 >= q_len) return;  // uniform: tile past this request's queries
    const int k_len_req = cu_k[req + 1] - cu_k[req];
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
    const int row = w * 32 + r;   // row of the workgroup this lane owns
    const int tok = tok0 + row / G;
    const int head = hkv * G + row % G;
    // with a group size that does not divide the rows (3, 5, 6, 7) the last rows past
    // TOK whole tokens are idle: they would belong to the next workgroup's first token
    constexpr bool kAllRows = TOK * G == kPrefillRows;
    const bool row_ok = tok < q_len && (kAllRows || row < TOK * G);
    // last key each row may see (the causal limit and the request's end)
    const int row_limit = min(causal ? cached + tok : k_len - 1, kv_end - 1);
    const int wave_first = min(tok0 + (w * 32) / G, q_len - 1);
    const int wave_last = min(tok0 + (kAllRows ? w * 32 + 31 : min(w * 32 + 31, TOK * G - 1)) / G, q_len - 1);
    const int wave_lo = min(causal ? cached + wave_first : k_len - 1, kv_end - 1);  // all rows see keys <= this
    // no row sees keys > this; -1 for a wave whose rows all lie past the request's queries
    // (the last query tile of a request, a one-token request): it only stages K/V
    const bool wave_rows = tok0 + (w * 32) / G < q_len;
    const int wave_hi = wave_rows ? min(causal ? cached + wave_last : k_len - 1, kv_end - 1) : -1;

    // q row of this lane, pieces 16s + 8h .. +8 of the head dim
    bf16x8_t qf[KS];
    {
        const uint16_t* qrow = q + (static_cast<int64_t>(q0 + tok) * num_heads + head) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok) u = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * h);
            qf[s] = __builtin_bit_cast(bf16x8_t, u);
        }
    }

    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[db][x] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int32_t* table_row = kPaged ? block_table + static_cast<int64_t>(req) * max_blocks : nullptr;
    const int64_t key_base = kPaged ? 0 : cu_k[req];  // first packed row of the request (contiguous)
    const int32_t row_stride = num_kv_heads * D * 2;  // bytes per slot

    // Loader.  Wave w stages keys [16w, 16w+16) of every tile; they lie in one page, so
    // the page's address is a scalar and each thread's offsets inside it never change.
    // Thread (c, g) of the wave loads chunk c (8 dims) of the KPT consecutive keys
    // g*KPT .. g*KPT+KPT-1, which lets it transpose V on its own: for every dim, the
    // KPT values are adjacent in a V^T row.  A buffer descriptor bounded to the wave's
    // valid keys makes every other load return zeros (keys past kv_end, and the whole
    // slice of a block id outside the pool), so nothing masked can be NaN.
    const int lc = lane / GPW;            // chunk of the row
    const int lg = lane % GPW;            // key group inside the wave's slice
    int32_t voff[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) voff[u] = (lg * KPT + u) * row_stride + lc * 16;
    const int64_t head_off = static_cast<int64_t>(hkv) * D * 2;

    // Block ids of a tile's pages come from one vector load (all lanes read the same
    // words), issued a tile ahead together with the K/V loads so the wait that precedes
    // the LDS stores covers it; scalar loads would instead hold up the next LDS wait,
    // which shares their counter.  The words are moved to scalar registers when used.
    constexpr int PAGES = BN / PBS;
    const __amdgpu_buffer_rsrc_t table_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(kPaged ? table_row : cu_k), 0, kPaged ? max_blocks * 4 : 0,
        kBufferDword3);
    auto load_ids = [&](int t) -> u32x4 {  // ids of tile t's pages; zero past the table
        const int off = t * PAGES * 4;
        if constexpr (!kPaged) {
            return u32x4{0, 0, 0, 0};
        } else if constexpr (PAGES == 4) {
            return __builtin_amdgcn_raw_buffer_load_b128(table_rsrc, off, 0, 0);
        } else if constexpr (PAGES == 2) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b64(table_rsrc, off, 0, 0);
            return u32x4{x[0], x[1], 0, 0};
        } else {
            return u32x4{__builtin_amdgcn_raw_buffer_load_b32(table_rsrc, off, 0, 0), 0, 0, 0};
        }
    };
    struct TileIds {
        uint32_t bits;  // bit i: page i is past kv_end or holds a block id inside the pool
        int32_t wave;   // block id of this wave's slice
    };
    auto scalar_ids = [&](int t, const u32x4& v) {
        TileIds r{1u, 0};
        if constexpr (kPaged) {
            r.bits = 0;
#pragma unroll
            for (int i = 0; i < PAGES; ++i) {
                const int32_t id = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(v[i]));
                const bool past = t * BN + i * PBS >= kv_end;
                r.bits |= (past || static_cast<uint32_t>(id) < static_cast<uint32_t>(num_blocks) ? 1u : 0u) << i;
                if ((WAVE_KEYS * w) / PBS == i) r.wave = id;
            }
        }
        return r;
    };
    uint4 kr[KPT], vr[KPT];
    auto fetch = [&](int t, int32_t id) {
        const int kw0 = t * BN + WAVE_KEYS * w;            // first key of this wave's slice
        const int nvalid = min(max(kv_end - kw0, 0), WAVE_KEYS);
        bool ok = nvalid > 0;
        int64_t base;
        if constexpr (kPaged) {
            ok = ok && static_cast<uint32_t>(id) < static_cast<uint32_t>(num_blocks);
            base = (static_cast<int64_t>(id) * PBS + kw0 % PBS) * row_stride + head_off;
        } else {
            base = (key_base + kw0) * row_stride + head_off;
        }
        if (!ok) base = 0;
        // (readfirstlane: a value the compiler forms on the vector unit would otherwise turn
        // each load into a loop over lanes)
        const int32_t bytes = __builtin_amdgcn_readfirstlane(ok ? nvalid * row_stride : 0);
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(k_cache + base), 0, bytes, kBufferDword3);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(v_cache + base), 0, bytes, kBufferDword3);
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            kr[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(krs, voff[u], 0, 0));
            vr[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(vrs, voff[u], 0, 0));
        }
    };

    // ids of tile t + 1 are loaded during tile t - 1 and used during tile t
    u32x4 ids_next = u32x4{0, 0, 0, 0};
    uint32_t ok_cur = 0;
    if (t_hi > t_lo) {
        const TileIds first = scalar_ids(t_lo, load_ids(t_lo));
        fetch(t_lo, first.wave);
        ok_cur = first.bits;
        if (t_hi - t_lo > 1) ids_next = load_ids(t_lo + 1);
    }
    // registers -> LDS buffer b for the tile whose loads are in kr / vr
    auto stage = [&](int b) {
            {
                // K rows as they are; V^T rows: for dim 8lc + e, this thread's KPT keys, at the
                // position of their 4-key quad q in the group's order q0 q2 q1 q3
                const int key0 = WAVE_KEYS * w + lg * KPT;
    #pragma unroll
                for (int u = 0; u < KPT; ++u)
                    *reinterpret_cast<uint4*>(&k_lds_all[b][(key0 + u) * PITCH + lc * 8]) = kr[u];
                const int quad = (lg * KPT) / 4;
                const int col = WAVE_KEYS * w + (quad & 1) * 8 + (quad >> 1) * 4 + (lg * KPT) % 4;
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
                    const int i = e / 2;
                    uint32_t* dst = reinterpret_cast<uint32_t*>(&v_lds_all[b][(lc * 8 + e) * PITCH_T + col]);
                    const uint32_t p01 = __builtin_amdgcn_perm(word(vr[1], i), word(vr[0], i), sel);
                    if constexpr (KPT == 4) {
                        const uint32_t p23 = __builtin_amdgcn_perm(word(vr[3], i), word(vr[2], i), sel);
                        if constexpr (PITCH_T % 4 == 0) {
                            *reinterpret_cast<uint2*>(dst) = make_uint2(p01, p23);
                        } else {  // rows only 4-byte aligned
                            dst[0] = p01;
                            dst[1] = p23;
                        }
                    } else {
                        *dst = p01;
                    }
                }
            }
    };
    // one tile from LDS buffer b: scores, online softmax, and the P V products
    auto compute = [&](int t, int b, uint32_t page_ok) {
        const int j0 = t * BN;
        const bool tile_ok = page_ok == (1u << PAGES) - 1;

        // S^T blocks: keys j0 + 32kb + (8i + 4h + jj), query row = this lane's row
        // The two 32-key blocks alternate, so consecutive products are independent, and
        // the K operands are read LDS_AHEAD products before their use.
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) s[kb][x] = 0.f;
        if constexpr (PA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(1);
        {
            constexpr int N = 2 * KS;
            auto read_k = [&](int o) {  // product o: k-step o / 2 of key block o % 2
                return *reinterpret_cast<const u16x8_t*>(&k_lds_all[b][((o % 2) * 32 + r) * PITCH + (o / 2) * 16 + 8 * h]);
            };
            u16x8_t kbuf[LDS_AHEAD];
#pragma unroll
            for (int o = 0; o < LDS_AHEAD; ++o) kbuf[o] = read_k(o);
#pragma unroll
            for (int o = 0; o < N; ++o) {
                const u16x8_t a = kbuf[o % LDS_AHEAD];
                if (o + LDS_AHEAD < N) kbuf[o % LDS_AHEAD] = read_k(o + LDS_AHEAD);
                s[o % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qf[o / 2], s[o % 2], 0, 0, 0);
            }
            pipeline_order<N, LDS_AHEAD>();
        }
        if constexpr (PA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(0);

        // scale to base 2, mask, running max
        const bool need_mask = !tile_ok || j0 + BN - 1 > wave_lo;
        const int lim = row_limit - j0;  // keys of this tile with index <= lim are visible
        // qscale > 0, so the max of the raw scores scales to the max of the scaled ones.
        // Masking (wave-uniform branches): keys past a row's limit always; keys of an
        // unassigned block only in the rare tile that has one.
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int key = kb * 32 + 8 * (x / 4) + 4 * h + (x % 4);
                    s[kb][x] = key <= lim ? s[kb][x] : -INFINITY;
                }
            if (!tile_ok) {
                // accumulator (kb, x) holds key 32kb + 8(x/4) + 4h + x%4; its page is
                // (32kb + 8(x/4)) / BS for both lane halves, a compile-time index
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int x = 0; x < 16; ++x) {
                        const int page = (kb * 32 + 8 * (x / 4)) / PBS;
                        s[kb][x] = (page_ok >> page) & 1u ? s[kb][x] : -INFINITY;
                    }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = fmaxf(mx, s[kb][x]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * qscale;
        // The reference max moves only when the tile's max exceeds it by more than
        // kRescaleSlack (base 2): the quotient sum(e^(s-m) v) / sum(e^(s-m)) does not depend
        // on m, and a stale m keeps every weight below 2^kRescaleSlack, so O and l are
        // rescaled in few tiles instead of nearly every one.
        const float m_new = mx > m + kRescaleSlack ? mx : m;
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float corr = __builtin_amdgcn_exp2f(m - m_use);
        float psum = 0.f;
        bf16x8_t pb[4];  // P^T operand of k-step ks: accumulators x = 8(ks%2) .. +8 of block ks/2
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[ks / 2][8 * (ks % 2) + e], qscale, -m_use));
                psum += p;
                pb[ks][e] = static_cast<__bf16>(p);
            }
        }
        l = l * corr + psum;
        m = m_new;
        if (__builtin_amdgcn_read_exec() & __ballot(corr != 1.f)) {  // some row's max moved
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int x = 0; x < 16; ++x) acc[db][x] *= corr;
        }

        // O^T += V^T P^T: A = V^T rows d = 32db + r, keys 16ks + 4h + (e%4) + 8(e/4),
        // stored contiguously at 16ks + 8h (quads h and 2 + h)
        // (products alternate over the DB accumulators; operands read LDS_AHEAD ahead)
        if constexpr (PA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(1);
        {
            constexpr int N = 4 * DB;
            auto read_v = [&](int o) {  // product o: k-step o / DB of dim block o % DB
                const uint32_t* src = reinterpret_cast<const uint32_t*>(
                    &v_lds_all[b][(32 * (o % DB) + r) * PITCH_T + 16 * (o / DB) + 8 * h]);
                uint2 lo, hi;
                if constexpr (PITCH_T % 4 == 0) {
                    lo = *reinterpret_cast<const uint2*>(src);
                    hi = *reinterpret_cast<const uint2*>(src + 2);
                } else {  // rows only 4-byte aligned
                    lo = make_uint2(src[0], src[1]);
                    hi = make_uint2(src[2], src[3]);
                }
                return __builtin_bit_cast(u16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
            };
            u16x8_t vbuf[LDS_AHEAD];
#pragma unroll
            for (int o = 0; o < LDS_AHEAD; ++o) vbuf[o] = read_v(o);
#pragma unroll
            for (int o = 0; o < N; ++o) {
                const u16x8_t a = vbuf[o % LDS_AHEAD];
                if (o + LDS_AHEAD < N) vbuf[o % LDS_AHEAD] = read_v(o + LDS_AHEAD);
                acc[o % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), pb[o / DB], acc[o % DB], 0, 0, 0);
            }
            pipeline_order<N, LDS_AHEAD>();
        }
        if constexpr (PA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(0);
    };

    // one barrier per tile: tile t + 1 is staged into the other buffer after tile t
    // is computed, while the loads of tile t + 2 are issued
    uint32_t ok_pend = 0;
    if (t_hi > t_lo) {
        __syncthreads();  // the orders staged in the K tile buffers are no longer read
        stage(0);
        if (t_hi - t_lo > 1) {
            const TileIds next = scalar_ids(t_lo + 1, ids_next);
            fetch(t_lo + 1, next.wave);
            ok_pend = next.bits;
            if (t_hi - t_lo > 2) ids_next = load_ids(t_lo + 2);
        }
        __syncthreads();
    }
    for (int t = t_lo; t < t_hi; ++t) {
        const int b = (t - t_lo) & 1;
        if (t * BN <= wave_hi) compute(t, b, ok_cur);
        if (t + 1 < t_hi) {
            stage(b ^ 1);
            ok_cur = ok_pend;
            if (t + 2 < t_hi) {
                const TileIds next = scalar_ids(t + 2, ids_next);
                fetch(t + 2, next.wave);
                ok_pend = next.bits;
                if (t + 3 < t_hi) ids_next = load_ids(t + 3);
            }
        }
        __syncthreads();
    }

    // normalise and store: lane holds d = 32db + 8i + 4h + jj of its row
    const float lt = l + __shfl_xor(l, 32);
    if (kSplit && n_split_job > 1) {
        // one key range of a split job: the unnormalised O, the reference max m and l
        // of each row go to the workspace, for prefill_merge_kernel
        if (!row_ok) return;
        const int64_t unit =
            ((static_cast<int64_t>(req) * num_kv_heads + hkv) * n_qtiles + qtile) * n_split + split;
        float* prow = part_o + (unit * kPrefillRows + row) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                *reinterpret_cast<float4*>(prow + 32 * db + 8 * i4 + 4 * h) =
                    make_float4(acc[db][4 * i4], acc[db][4 * i4 + 1], acc[db][4 * i4 + 2], acc[db][4 * i4 + 3]);
        if (h == 0) part_ml[unit * kPrefillRows + row] = make_float2(m, lt);
        return;
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (!row_ok) return;
    uint16_t* orow = out + (static_cast<int64_t>(q0 + tok) * num_heads + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            uint32_t lo = static_cast<uint32_t>(to_bf16_bits(acc[db][4 * i4 + 0] * inv)) |
                          (static_cast<uint32_t>(to_bf16_bits(acc[db][4 * i4 + 1] * inv)) << 16);
            uint32_t hi = static_cast<uint32_t>(to_bf16_bits(acc[db][4 * i4 + 2] * inv)) |
                          (static_cast<uint32_t>(to_bf16_bits(acc[db][4 * i4 + 3] * inv)) << 16);
            *reinterpret_cast<uint2*>(orow + 32 * db + 8 * i4 + 4 * h) = make_uint2(lo, hi);
        }
}

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
// for fp32 pools.
int prefill_by_token(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                     int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                     int32_t max_seqlen_q, const int32_t* block_table, int32_t max_blocks,
                     float scale, int32_t causal, hipStream_t s, int32_t contiguous);

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
constexpr int64_t kMinSplitTiles = 16;
constexpr int64_t kMinSplitTilesExact = 8;

struct SplitPlan {
    int32_t n_split;      // key ranges per job at most (1: no split)
    int32_t split_tiles;  // key tiles per range (the last range of a job takes the rest)
    int64_t units;        // dense jobs x n_split: rows of the workspace
};

// workgroup slots of the current device: two per CU (the prefill kernel's occupancy).
// The CU count is read once per device (each device of a process has its own entry).
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

template <int D, int G, int BS>
int launch_prefill(const KvSource& kv, void* out, const void* q, int32_t batch,
                   int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                   int32_t max_seqlen_q, float scale, int32_t causal, hipStream_t stream,
                   const SplitPlan& sp, void* workspace, int passes) {
    const int tok_per_wg = kPrefillRows / G;
    const int64_t n_qtiles = (max_seqlen_q + tok_per_wg - 1) / tok_per_wg;
    const int64_t n_groups = static_cast<int64_t>(kv.num_kv_heads) * batch;
    const int64_t padded = (n_groups + kXcds - 1) / kXcds * n_qtiles * sp.n_split * kXcds;
    if (padded > INT32_MAX) return PA_ERR_UNSUPPORTED;
    float* part_o = sp.n_split > 1 ? static_cast<float*>(workspace) : nullptr;
    float2* part_ml = sp.n_split > 1
        ? reinterpret_cast<float2*>(part_o + static_cast<size_t>(sp.units) * kPrefillRows * D) : nullptr;
    const dim3 grid(static_cast<uint32_t>(padded));
    if (!(passes & kPass1)) {
        // the merge alone (of ranges stored by an earlier call)
    } else if (sp.n_split > 1)
        hipLaunchKernelGGL((prefill_kernel<D, G, BS, true>), grid, dim3(kPrefillThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const char*>(kv.k),
                           static_cast<const char*>(kv.v), cu_q, cu_k, kv.table,
                           static_cast<uint16_t*>(out), num_heads, kv.num_kv_heads,
                           kv.num_blocks, kv.max_blocks, scale * kLog2e, causal,
                           static_cast<int32_t>(n_qtiles), static_cast<int32_t>(n_groups),
                           sp.n_split, sp.split_tiles, part_o, part_ml);
    else
        hipLaunchKernelGGL((prefill_kernel<D, G, BS, false>), grid, dim3(kPrefillThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const char*>(kv.k),
                           static_cast<const char*>(kv.v), cu_q, cu_k, kv.table,
                           static_cast<uint16_t*>(out), num_heads, kv.num_kv_heads,
                           kv.num_blocks, kv.max_blocks, scale * kLog2e, causal,
                           static_cast<int32_t>(n_qtiles), static_cast<int32_t>(n_groups), 1, 0,
                           nullptr, nullptr);
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

template <int D>
int dispatch_prefill_group(int G, const KvSource& kv, void* out, const void* q, int32_t batch,
                           int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                           int32_t max_seqlen_q, float scale, int32_t causal,
                           hipStream_t stream, const SplitPlan& sp, void* workspace, int passes) {
#define PA_PREFILL_LAUNCH(GG, BB) \
    launch_prefill<D, GG, BB>(kv, out, q, batch, num_heads, cu_q, cu_k, max_seqlen_q, scale, causal, stream, sp, workspace, passes)
#define PA_PREFILL_CASE(GG)                                                                     \
    case GG:                                                                                    \
        if (!kv.paged) return PA_PREFILL_LAUNCH(GG, 0);                              \
        return kv.block_size == 16 ? PA_PREFILL_LAUNCH(GG, 16) : PA_PREFILL_LAUNCH(GG, 32);
    switch (G) {
        PA_PREFILL_CASE(1)
        PA_PREFILL_CASE(2)
        PA_PREFILL_CASE(3)
        PA_PREFILL_CASE(4)
        PA_PREFILL_CASE(5)
        PA_PREFILL_CASE(6)
        PA_PREFILL_CASE(7)
        PA_PREFILL_CASE(8)
        PA_PREFILL_CASE(16)
        PA_PREFILL_CASE(32)
        default: return PA_ERR_UNSUPPORTED;
    }
#undef PA_PREFILL_CASE
#undef PA_PREFILL_LAUNCH
}

int prefill_impl(const KvSource& kv, int32_t head_dim, void* out, const void* q, int32_t batch,
                 int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                 int32_t max_seqlen_q, float scale, int32_t causal, hipStream_t s,
                 const SplitPlan& sp = SplitPlan{1, 0, 0}, void* workspace = nullptr,
                 int passes = kPass1 | kPass2) {
    if (num_heads % kv.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || scale == INFINITY) return PA_ERR_INVALID_ARG;
    const int G = num_heads / kv.num_kv_heads;
    if (head_dim == 128)
        return dispatch_prefill_group<128>(G, kv, out, q, batch, num_heads, cu_q, cu_k,
                                           max_seqlen_q, scale, causal != 0, s, sp, workspace,
                                           passes);
    if (head_dim == 64)
        return dispatch_prefill_group<64>(G, kv, out, q, batch, num_heads, cu_q, cu_k,
                                          max_seqlen_q, scale, causal != 0, s, sp, workspace,
                                          passes);
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

// Key ranges: of partition_tokens keys (rounded up to whole 64-key tiles) when given.
// Else ranges long enough for about kDecodeTargetUnits (job, range) units over the
// longest sequence, of at least kDecodeMinSplitTiles tiles, and of up to kDecodeSplitTiles
// while that still leaves kDecodeFewUnits units: a decode job has one query row per head,
// so a range's fixed costs weigh more than in a prefill.  (Measured on 64 query / 8 or 4
// KV heads: 4 sequences of 16K keys and 16 of 8K ran fastest in ranges of 12-16 tiles,
// 64 sequences of 4K in two ranges rather than four, 8 of 40K in 16 ranges of 40 tiles;
// 8 sequences of 4K with 40 / 8 heads in ranges of 8 tiles, 29 against 37 us at 16.)
constexpr int64_t kDecodeTargetUnits = 1024;
constexpr int64_t kDecodeFewUnits = 512;
constexpr int64_t kDecodeMinSplitTiles = 8;
constexpr int64_t kDecodeSplitTiles = 32;

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
