// Varlen (packed) paged prefill on the matrix cores: the kernel.
//
// What it computes ("从零开始写Qwen3（六）PagedAttention", fast-attn 库的使用: the varlen call
// with a block table; "Sayfalı dikkat", Değişken uzunluklu yol): request i owns query
// rows [cu_q[i], cu_q[i+1]) of the packed q and k_len = cu_k[i+1] - cu_k[i] keys, read
// through block_table row i ("Paged attention 与 online softmax" §11.1).  With
// c = k_len - q_len cached tokens, query row t sees keys j <= c + t when causal.
//
// How (gfx950, bf16 in, fp32 accumulate):
// * A workgroup is a job: 128 "rows" of one request and one KV head, a row being a
//   (token, query head) pair with the G query heads of the KV head next to each other, so
//   every K/V tile read serves all of them.  Two waves of 64 rows (two 32-row blocks)
//   each, one wave per SIMD and two workgroups per CU: every K or V^T operand read from
//   LDS feeds the products of both row blocks, which halves the LDS bytes per product
//   against one 32-row block per wave.
// * Keys are walked in tiles of 32, FlashAttention-style ("结合nanovllm的FlashAttention和
//   PagedAttention主要原理概述" 题目3): each tile is gathered through the block table into LDS,
//   its scores are folded into the running (m, l, O) with the §11.2 rule, and O is
//   normalised once at the end.
// * Transposed products keep a query row inside one lane: S^T = K Q^T with
//   v_mfma_f32_32x32x16_bf16 (A = a K row per lane from LDS, B = the lane's q row held in
//   registers), so lane l holds 16 of the tile's scores for row l%32 (the other 16 sit in
//   lane l^32).  O^T += V^T P^T takes P straight from the S^T accumulators: the key order
//   inside each 16-key step is permuted the same way on both operands, and the loader
//   stores V transposed in that order, so a V^T operand is 16 contiguous bytes.
// * Software pipeline, one barrier per tile: while the products of tile t+1's scores run,
//   the wave computes tile t's weights on the vector unit (the two are independent, and
//   one wave issues vector instructions while its matrix products execute), then the
//   products of tile t's P V.  The tiles live in a ring of three LDS buffers: t is read
//   for V, t+1 for K, t+2 is being written from registers, whose loads for t+3 are in
//   flight.
// * Weights without a per-tile maximum: p = 2^(s*scale*log2e - m) against the row's
//   reference m, which moves only on a rare slow path (the first tile a row sees, or a
//   tile whose weights sum past 2^64).  The quotient sum(p v) / sum(p) does not depend on
//   m, and the bound keeps every sum finite.  Row sums are taken from the bf16 weights
//   that enter the products (v_dot2).
// * Each wave stages a 16-key slice of every tile, which lies in one page, so the page
//   address is a scalar; buffer loads bounded to the slice's valid keys return zeros past
//   kv_end and for a block id outside the pool, so masked keys never bring NaN into a
//   product.  Masking sets scores past a row's limit (and of unassigned blocks) to -inf.
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

constexpr int kPrefillWaves = 2;                          // waves per workgroup
constexpr int kWaveRows = 64;                             // rows per wave (two 32-row blocks)
constexpr int kPrefillRows = kPrefillWaves * kWaveRows;   // rows per workgroup (a job)
constexpr int kPrefillKeys = 32;                          // keys per tile
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kPrefillStages = 3;                         // LDS tile buffers
constexpr int kXcds = 8;            // accelerator complex dies of an MI355X
constexpr float kFastSumLimit = 18446744073709551616.f;  // 2^64: weights of a tile on the fast path
constexpr int kMaxRankedRequests = 256;  // requests ordered by key count in-kernel
// Jobs per XCD ordered by key tiles in-kernel.  Ranking costs O(jobs^2) LDS compares per
// workgroup and separates the query tiles of a group (which then stop sharing K/V pages
// in L2); past a few jobs per workgroup slot the batch order, which keeps a group's tiles
// together, measured faster.
constexpr int kMaxRankedJobs = 384;

// Key ranges of a job of `tiles` key tiles when jobs are cut into ranges of split_tiles
// tiles, at most n_split of them (the last one takes the rest).
__host__ __device__ inline int split_count(int tiles, int n_split, int split_tiles) {
    if (n_split <= 1 || tiles <= split_tiles) return 1;
    const int parts = (tiles + split_tiles - 1) / split_tiles;
    return parts < n_split ? parts : n_split;
}

// Row of V^T dimension i in LDS.  Rows 8 apart would share banks when the loader writes
// them (a thread writes the 8 dims of one 16-byte chunk); XOR-ing the low two bits with
// bits 3-4 spreads them, and 16 consecutive dims (one operand read) stay conflict free.
__device__ __forceinline__ int vt_row(int i) { return i ^ ((i >> 3) & 3); }

constexpr bf16x2_t kOnes2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

// sched_group_barrier masks
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100, kSgDsWrite = 0x200;

// BS = 0: contiguous K/V.  kSplit: jobs may be cut into key ranges (n_split, split_tiles);
// without it those arguments are ignored and the kernel is the plain one.
template <int D, int G, int BS, bool kSplit>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_kernel(
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
    constexpr int PBS = kPaged ? BS : BN;       // keys per page (one page per tile when contiguous)
    constexpr int PAGES = BN / PBS;             // pages of a tile (1 or 2)
    constexpr int TOK = kPrefillRows / G;       // tokens per workgroup
    constexpr int KS = D / 16;                  // MFMA k-steps over the head dim
    constexpr int DB = D / 32;                  // 32-wide blocks of the head dim in O^T
    constexpr int CHUNKS = D / 8;               // 16-byte pieces per K/V row
    constexpr int SLICE = BN / kPrefillWaves;   // keys of a tile staged by each wave
    constexpr int GPW = kWave / CHUNKS;         // key groups per wave
    constexpr int KPT = SLICE / GPW;            // keys per loader thread: 4 (d 128), 2 (d 64)
    static_assert(KPT == 2 || KPT == 4, "loader split");
    static_assert(PBS % SLICE == 0 && BN % PBS == 0, "a wave's keys lie in one page");
    // LDS: K rows with a 16-byte pad (16 consecutive rows then cover all banks once, for
    // the operand reads and the loader's writes alike); V^T rows of 32 keys, 16-byte pad
    constexpr int KP = D + 8;                   // K row pitch (elements)
    constexpr int VP = BN + 8;                  // V^T row pitch (elements)
    constexpr int K_ELEMS = BN * KP;
    constexpr int STAGE = K_ELEMS + D * VP;     // one tile buffer
    __shared__ __align__(16) uint16_t lds[kPrefillStages * STAGE];
    static_assert(2 * kMaxRankedRequests + kMaxRankedJobs <= K_ELEMS / 2,
                  "the ranking tables fit in the first K tile buffer");

    // Work items are jobs (group, query tile), a group being one (request, KV head).
    // Workgroup L runs on XCD L % 8 (workgroups are handed to the XCDs round-robin), and
    // the jobs of group g all run on XCD g % 8: the query tiles of a group read the same
    // K/V pages, which then stay in that XCD's L2.  Requests are ranked by key count,
    // longest first, and group g belongs to the request of rank g / Hkv, so that every
    // request's heads are spread over the 8 XCDs.  Within an XCD the jobs start in order
    // of decreasing key-tile count (longest-processing-time first): workgroup slot s of
    // the XCD takes the job of rank s, and the short jobs fill the gaps at the end.
    // Every workgroup derives the same orders from cu_q / cu_k in LDS (the first tile
    // buffer, overwritten only after a barrier); beyond kMaxRankedRequests requests or
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
    int32_t* const perm = reinterpret_cast<int32_t*>(lds);           // request of each rank
    int32_t* const klen = perm + kMaxRankedRequests;                 // key count of each request
    int32_t* const jobs = klen + kMaxRankedRequests;                 // key tiles of each job
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
    // with a group size that does not divide the rows (3, 5, 6, 7) the last rows past
    // TOK whole tokens are idle: they would belong to the next workgroup's first token
    constexpr bool kAllRows = TOK * G == kPrefillRows;
    constexpr int kUsedRows = TOK * G;
    // the two rows of this lane: row block rb holds workgroup row 64w + 32rb + r
    int tok[2], head[2], row_limit[2];
    bool row_ok[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
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
    bf16x8_t qf[2][KS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const uint16_t* qrow = q + (static_cast<int64_t>(q0 + tok[rb]) * num_heads + head[rb]) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row_ok[rb]) u = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * h);
            qf[rb][s] = __builtin_bit_cast(bf16x8_t, u);
        }
    }

    f32x16_t acc[2][DB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int x = 0; x < 16; ++x) acc[rb][db][x] = 0.f;
    float m_ref[2] = {-INFINITY, -INFINITY};  // row reference (base 2, scaled); same in lanes l, l^32
    float lsum[2] = {0.f, 0.f};               // this lane's part of the row sums

    const int32_t* table_row = kPaged ? block_table + static_cast<int64_t>(req) * max_blocks : nullptr;
    const int64_t key_base = kPaged ? 0 : cu_k[req];  // first packed row of the request (contiguous)
    const int32_t row_stride = num_kv_heads * D * 2;  // bytes per slot

    // Loader.  Wave w stages keys [16w, 16w+16) of every tile; they lie in one page, so
    // the page's address is a scalar and each thread's offsets inside it never change.
    // Thread (c, g) of the wave loads chunk c (8 dims) of the KPT consecutive keys
    // g*KPT .. g*KPT+KPT-1, which lets it transpose V on its own: for every dim, the KPT
    // values are adjacent in a V^T row.  A buffer descriptor bounded to the wave's valid
    // keys makes every other load return zeros (keys past kv_end, and the whole slice of
    // a block id outside the pool), so nothing masked can be NaN.
    const int lc = lane / GPW;            // chunk of the row
    const int lg = lane % GPW;            // key group inside the wave's slice
    int32_t voff[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) voff[u] = (lg * KPT + u) * row_stride + lc * 16;
    const int64_t head_off = static_cast<int64_t>(hkv) * D * 2;

    // Block ids of a tile's pages come from one vector load (all lanes read the same
    // words), issued with the K/V loads of the tile before, so the wait that precedes the
    // LDS stores covers it (scalar loads would hold up the LDS waits, which share their
    // counter).  The words are moved to scalar registers when used.
    const __amdgpu_buffer_rsrc_t table_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(kPaged ? table_row : cu_k), 0, kPaged ? max_blocks * 4 : 0,
        kBufferDword3);
    auto load_ids = [&](int t) -> u32x4 {  // ids of tile t's pages; zero past the table
        const int off = t * PAGES * 4;
        if constexpr (!kPaged) {
            return u32x4{0, 0, 0, 0};
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
        TileIds res{(1u << PAGES) - 1, 0};
        if constexpr (kPaged) {
            res.bits = 0;
#pragma unroll
            for (int i = 0; i < PAGES; ++i) {
                const int32_t id = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(v[i]));
                const bool past = t * BN + i * PBS >= kv_end;
                res.bits |= (past || static_cast<uint32_t>(id) < static_cast<uint32_t>(num_blocks) ? 1u : 0u) << i;
                if ((SLICE * w) / PBS == i) res.wave = id;
            }
        }
        return res;
    };
    uint4 kr[KPT], vr[KPT];
    auto fetch_into = [&](int t, int32_t id, uint4 (&kd)[KPT], uint4 (&vd)[KPT]) {
        const int kw0 = t * BN + SLICE * w;                // first key of this wave's slice
        const int nvalid = min(max(kv_end - kw0, 0), SLICE);
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
            kd[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(krs, voff[u], 0, 0));
            vd[u] = to_uint4(__builtin_amdgcn_raw_buffer_load_b128(vrs, voff[u], 0, 0));
        }
    };
    // registers -> LDS buffer b, in units: unit u < KPT stores K row u of this thread as it
    // is; unit KPT + e stores dim 8lc + e of V^T: this thread's KPT keys at the position
    // of their 4-key quad q in the group's order q0 q2 q1 q3 (the order in which the P^T
    // operand holds them)
    constexpr int kStageUnits = KPT + 8;
    const int k_st = (SLICE * w + lg * KPT) * KP + lc * 8;
    const int quad = (lg * KPT) / 4;
    const int v_col = SLICE * w + (quad & 1) * 8 + (quad >> 1) * 4 + (lg * KPT) % 4;
    auto stage_unit = [&](int b, int j, const uint4 (&ks_)[KPT], const uint4 (&vs_)[KPT]) {
        uint16_t* const kb = lds + b * STAGE;
        uint16_t* const vb = kb + K_ELEMS;
        if (j < KPT) {
            *reinterpret_cast<uint4*>(kb + k_st + j * KP) = ks_[j];
            return;
        }
        const int e = j - KPT;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
        const int i = e / 2;
        uint16_t* dst = vb + vt_row(lc * 8 + e) * VP + v_col;
        const uint32_t p01 = __builtin_amdgcn_perm(word(vs_[1], i), word(vs_[0], i), sel);
        if constexpr (KPT == 4) {
            const uint32_t p23 = __builtin_amdgcn_perm(word(vs_[3], i), word(vs_[2], i), sel);
            *reinterpret_cast<uint2*>(dst) = make_uint2(p01, p23);
        } else {
            *reinterpret_cast<uint32_t*>(dst) = p01;
        }
    };
    auto stage_from = [&](int b, const uint4 (&ks_)[KPT], const uint4 (&vs_)[KPT]) {
#pragma unroll
        for (int j = 0; j < kStageUnits; ++j) stage_unit(b, j, ks_, vs_);
    };

    // MFMA operand reads.  K: key r of the tile, dims 16ks + 8h .. +8.  V^T: dim
    // 32db + r, keys 16ks + 8h .. +8 in the permuted order.
    const int k_rd = r * KP + 8 * h;
    const int v_rd = K_ELEMS + vt_row(r) * VP + 8 * h;   // vt_row(32db + r) = 32db + vt_row(r)
    auto read_k = [&](int b, int ks) {
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(lds + b * STAGE + k_rd + 16 * ks));
    };
    auto read_v = [&](int b, int db, int ks) {
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u16x8_t*>(
            lds + b * STAGE + v_rd + 32 * db * VP + 16 * ks));
    };

    // S^T of a tile: s[rb] accumulates keys 8(x/4) + 4h + x%4 of the tile for row block rb
    auto zero_s = [&](f32x16_t (&s)[2]) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int x = 0; x < 16; ++x) s[rb][x] = 0.f;
    };
    auto qk = [&](int b, f32x16_t (&s)[2]) {
        zero_s(s);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t a = read_k(b, ks);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[0][ks], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[1][ks], s[1], 0, 0, 0);
        }
    };
    // References.  Each row's reference is the maximum of its scores in the unit's first
    // tile (0 for a row with no visible key there), and the weights exp2(s - reference)
    // are never rescaled, so O is touched by nothing but the matrix products.  A later
    // score far above the reference shows as a tile's weight sum above 2^64 (or not
    // finite); the workgroup then flags the unit and computes it again, first the exact
    // row maxima (a pass over the scores alone), then the attention against them.
    __shared__ int32_t redo;
    // one of the 16 pair sums of a tile's weights (pair o: row block o / 8, k-step
    // (o / 4) % 2, elements 2(o % 4), +1), into one of two partial sums per row block
    auto pair_sum = [&](const bf16x8_t (&pb)[2][2], int o, float (&part)[2][2]) {
        const int rb = o / 8, ks = (o / 4) % 2, e = 2 * (o % 4);
        const bf16x2_t pp = {pb[rb][ks][e], pb[rb][ks][e + 1]};
        part[rb][o % 2] = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, part[rb][o % 2], false);
    };
    // Tile t+1's score products (K from buffer b) with tile t's weights (scores sc) in
    // between, in source order: per k-step, its two products, then a share of the weights
    // (32 per lane over the KS steps).  sched_barrier(0) fences keep each share next to its
    // products: the products run on the matrix cores while the wave issues the vector
    // instructions.  Nothing here waits on a weight (the row sums, which would, are taken
    // during the P V products), so the wave never stalls behind an exponential.
    auto qk_softmax = [&](int b, const f32x16_t (&sc)[2], f32x16_t (&sn)[2], bf16x8_t (&pb)[2][2]) {
        constexpr int VPC = 32 / KS;  // weights per k-step: 4 (d 128) or 8 (d 64)
        zero_s(sn);
        const float mu[2] = {m_ref[0], m_ref[1]};
        bf16x8_t a[KS];
        a[0] = read_k(b, 0);
        a[1] = read_k(b, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) a[ks + 2] = read_k(b, ks + 2);
            sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[0][ks], sn[0], 0, 0, 0);
            sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[1][ks], sn[1], 0, 0, 0);
#pragma unroll
            for (int v = ks * VPC; v < (ks + 1) * VPC; v += 2) {
                const int rb = v / 16, x = v % 16;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[rb][x], qscale, -mu[rb]));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[rb][x + 1], qscale, -mu[rb]));
                const bf16x2_t pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
                pb[rb][x / 8][x % 8] = pp[0];
                pb[rb][x / 8][x % 8 + 1] = pp[1];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Tile t's P V products (V^T from buffer b) with the staging of tile t+2 into buffer
    // b2 in between: per operand read, its two products, then a share of the LDS stores.
    // The row sums of the weights are taken here too, two independent partial sums per row
    // block; a tile whose sums are not finite and at most 2^64 (a score far above its row's
    // reference) flags the unit to be computed again against exact row maxima.
    auto pv_stage = [&](int b, const bf16x8_t (&pb)[2][2], int b2) {
        constexpr int NO = 2 * DB;  // V^T operands of a tile
        float part[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
        bf16x8_t va[NO];
        va[0] = read_v(b, 0, 0);
        va[1] = read_v(b, 1 % DB, 1 / DB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NO; ++i) {
            const int ks = i / DB, db = i % DB;
            if (i + 2 < NO) va[i + 2] = read_v(b, (i + 2) % DB, (i + 2) / DB);
            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[0][ks], acc[0][db], 0, 0, 0);
            acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pb[1][ks], acc[1][db], 0, 0, 0);
#pragma unroll
            for (int j = i; j < kStageUnits; j += NO) stage_unit(b2, j, kr, vr);
#pragma unroll
            for (int o = i; o < 16; o += NO) pair_sum(pb, o, part);
            __builtin_amdgcn_sched_barrier(0);
        }
        const float ps0 = part[0][0] + part[0][1], ps1 = part[1][0] + part[1][1];
        lsum[0] += ps0;
        lsum[1] += ps1;
        if (!(ps0 <= kFastSumLimit) || !(ps1 <= kFastSumLimit)) redo = 1;
    };

    // masking of tile t: keys past a row's limit, keys of an unassigned block (none
    // in most tiles: the caller tests need_mask first)
    auto need_mask = [&](int t, uint32_t page_ok) {
        return page_ok != (1u << PAGES) - 1 || t * BN + BN - 1 > wave_lo;
    };
    auto mask = [&](int t, f32x16_t (&s)[2], uint32_t page_ok) {
        const int j0 = t * BN;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
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
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int page = (8 * (x / 4)) / PBS;
                    s[rb][x] = (page_ok >> page) & 1u ? s[rb][x] : -INFINITY;
                }
        }
    };
    // weights of a tile against the current references: P^T operands pb[rb][ks] (keys of
    // k-step ks: accumulators 8ks .. 8ks+7).  Their row sums are taken with the P V
    // products (pv_stage), from the rounded weights that enter them.
    auto weights = [&](const f32x16_t (&s)[2], bf16x8_t (&pb)[2][2]) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[rb][8 * ks + e], qscale, -m_ref[rb]));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[rb][8 * ks + e + 1], qscale, -m_ref[rb]));
                    const bf16x2_t pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
                    pb[rb][ks][e] = pp[0];
                    pb[rb][ks][e + 1] = pp[1];
                }
    };
    // row maxima of a tile's scores (scaled to base 2; lanes l and l^32 agree)
    auto tile_max = [&](const f32x16_t (&s)[2], float (&mx)[2]) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float v = -INFINITY;
#pragma unroll
            for (int x = 0; x < 16; ++x) v = fmaxf(v, s[rb][x]);
            mx[rb] = fmaxf(v, __shfl_xor(v, 32)) * qscale;  // qscale > 0: the max scales with it
        }
    };
    // O stays in the accumulation registers: nothing but the products touches it until
    // the end
    auto pin_acc = [&]() {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(acc[rb][db]));
    };

    // ---- the key loop ---------------------------------------------------------------
    // One pass over the unit's tiles: the attention (MAX_ONLY false), or the row maxima
    // of the scores alone into m_ref (MAX_ONLY true).  Staging and loads run every
    // iteration: past the unit's last tile they load zeros (the descriptors' bounds) into
    // a buffer nobody reads.  The tiles this wave computes come first, two per loop trip
    // so that the two sets of score registers alternate without copies; the last one has
    // no next tile's products; tiles past the wave's rows (if any) are only staged.
    const int n = t_hi - t_lo;
    auto key_pass = [&](auto max_only, bool set_refs) {
        constexpr bool MAX_ONLY = decltype(max_only)::value;
        uint32_t okq = 0;  // page bits of tiles t, t+1, t+2, t+3 at bits 0, 2, 4, 6
        u32x4 ids_next = u32x4{0, 0, 0, 0};
        f32x16_t sa[2], sb[2];
        if (n <= 0) return;
        {
            // the first two tiles' ids, then their loads, in flight together
            const u32x4 id0 = load_ids(t_lo), id1 = load_ids(t_lo + 1);
            const TileIds first = scalar_ids(t_lo, id0), second = scalar_ids(t_lo + 1, id1);
            uint4 kr1[KPT], vr1[KPT];
            fetch_into(t_lo, first.wave, kr, vr);
            fetch_into(t_lo + 1, second.wave, kr1, vr1);
            ids_next = load_ids(t_lo + 2);
            okq = first.bits | (second.bits << 2);
            __syncthreads();  // LDS of the job orders or of the pass before: no longer read
            stage_from(0, kr, vr);
            stage_from(1, kr1, vr1);
            const TileIds t2 = scalar_ids(t_lo + 2, ids_next);
            fetch_into(t_lo + 2, t2.wave, kr, vr);
            okq |= t2.bits << 4;
            ids_next = load_ids(t_lo + 3);
            __syncthreads();
            if (t_lo < t_end) {
                qk(0, sa);
                asm volatile("" : "+v"(sa[0]), "+v"(sa[1]));
                if (!MAX_ONLY && set_refs) {
                    if (need_mask(t_lo, okq & 3u)) mask(t_lo, sa, okq & 3u);
                    float mx[2];
                    tile_max(sa, mx);
                    m_ref[0] = mx[0] == -INFINITY ? 0.f : mx[0];
                    m_ref[1] = mx[1] == -INFINITY ? 0.f : mx[1];
                }
            }
            if (!MAX_ONLY && set_refs && t_lo >= t_end) m_ref[0] = m_ref[1] = 0.f;
        }
        int b = 0;  // buffer of tile t
        // the loads of tile t+3 (after tile t+2 left the registers for LDS)
        auto fetch_next = [&](int t) {
            const TileIds ti = scalar_ids(t + 3, ids_next);
            fetch_into(t + 3, ti.wave, kr, vr);
            okq |= ti.bits << 6;
            ids_next = load_ids(t + 4);
        };
        auto advance = [&]() {
            __syncthreads();
            okq >>= 2;
            b = b == kPrefillStages - 1 ? 0 : b + 1;
        };
        // one computed tile t (scores in sc); NEXT: tile t+1's score products into sn
        auto step = [&](int t, f32x16_t (&sc)[2], f32x16_t (&sn)[2], auto next) {
            constexpr bool NEXT = decltype(next)::value;
            const int b1 = b == kPrefillStages - 1 ? 0 : b + 1;
            const int b2 = b == 0 ? kPrefillStages - 1 : b - 1;
            if (need_mask(t, okq & 3u)) mask(t, sc, okq & 3u);
            if constexpr (MAX_ONLY) {
                float mx[2];
                tile_max(sc, mx);
                m_ref[0] = fmaxf(m_ref[0], mx[0]);
                m_ref[1] = fmaxf(m_ref[1], mx[1]);
                if constexpr (NEXT) qk(b1, sn);
                stage_from(b2, kr, vr);
            } else {
                bf16x8_t pb[2][2];
                if constexpr (NEXT) {
                    qk_softmax(b1, sc, sn, pb);
                } else {
                    weights(sc, pb);
                }
                pv_stage(b, pb, b2);
                pin_acc();
            }
            fetch_next(t);
            // the next tile's scores are read by vector instructions: keep them in vector
            // registers (placed after the products of both tiles, so that it does not split
            // the stretch above)
            if constexpr (NEXT) asm volatile("" : "+v"(sn[0]), "+v"(sn[1]));
            advance();
        };
        int t = t_lo;
        for (; t + 2 < t_end; t += 2) {
            step(t, sa, sb, std::true_type{});
            step(t + 1, sb, sa, std::true_type{});
        }
        if (t + 1 < t_end) {
            step(t, sa, sb, std::true_type{});
            step(t + 1, sb, sa, std::false_type{});
            t += 2;
        } else if (t < t_end) {
            step(t, sa, sb, std::false_type{});
            t += 1;
        }
        for (; t < t_hi; ++t) {
            stage_from(b == 0 ? kPrefillStages - 1 : b - 1, kr, vr);
            fetch_next(t);
            advance();
        }
    };
    if (tid == 0) redo = 0;  // (seen by every wave after the pass's first barrier)
    pin_acc();
    key_pass(std::false_type{}, true);
    __syncthreads();  // every wave's flag is in
    if (redo) {       // uniform: the same LDS word for the whole workgroup
        // exact row maxima first, then the attention against them (no weight exceeds 1)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) m_ref[rb] = -INFINITY;
        key_pass(std::true_type{}, false);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
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
    for (int rb = 0; rb < 2; ++rb) {
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
        if (!row_ok[rb]) continue;
        uint16_t* orow = out + (static_cast<int64_t>(q0 + tok[rb]) * num_heads + head[rb]) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                uint32_t lo = static_cast<uint32_t>(to_bf16_bits(acc[rb][db][4 * i4 + 0] * inv)) |
                              (static_cast<uint32_t>(to_bf16_bits(acc[rb][db][4 * i4 + 1] * inv)) << 16);
                uint32_t hi = static_cast<uint32_t>(to_bf16_bits(acc[rb][db][4 * i4 + 2] * inv)) |
                              (static_cast<uint32_t>(to_bf16_bits(acc[rb][db][4 * i4 + 3] * inv)) << 16);
                *reinterpret_cast<uint2*>(orow + 32 * db + 8 * i4 + 4 * h) = make_uint2(lo, hi);
            }
    }
}

}  // namespace pa
