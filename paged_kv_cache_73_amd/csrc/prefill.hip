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

template <int D, int G, int BS>  // BS = 0: contiguous K/V
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    const uint16_t* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ block_table,
    uint16_t* __restrict__ out, int32_t num_heads, int32_t num_kv_heads, int32_t num_blocks,
    int32_t max_blocks, float qscale, int32_t causal, int32_t n_qtiles, int32_t n_groups) {
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
    const int n_jobs = (n_groups + kXcds - 1) / kXcds * n_qtiles;  // workgroups per XCD
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
    int group, qtile;
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
                const int g = (c / n_qtiles) * kXcds + xcd;
                const int tiles = g < n_groups ? job_tiles(request_of(g / num_kv_heads), (c % n_qtiles) * TOK) : -1;
                key = (min(tiles + 1, 0x7FFE) << 16) | (0xFFFF - c);
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
        group = (c / n_qtiles) * kXcds + xcd;
        qtile = c % n_qtiles;
    } else {
        // the groups of the XCD in turn, the query tiles of a group back to back, the
        // later ones (which see more keys under the causal mask) first
        group = (slot / n_qtiles) * kXcds + xcd;
        qtile = n_qtiles - 1 - slot % n_qtiles;
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
    const int wave_hi = min(causal ? cached + wave_last : k_len - 1, kv_end - 1);   // no row sees keys > this

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
    if (n_tiles > 0) {
        const TileIds first = scalar_ids(0, load_ids(0));
        fetch(0, first.wave);
        ok_cur = first.bits;
        if (n_tiles > 1) ids_next = load_ids(1);
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
    if (n_tiles > 0) {
        __syncthreads();  // the orders staged in the K tile buffers are no longer read
        stage(0);
        if (n_tiles > 1) {
            const TileIds next = scalar_ids(1, ids_next);
            fetch(1, next.wave);
            ok_pend = next.bits;
            if (n_tiles > 2) ids_next = load_ids(2);
        }
        __syncthreads();
    }
    for (int t = 0; t < n_tiles; ++t) {
        const int b = t & 1;
        if (t * BN <= wave_hi) compute(t, b, ok_cur);
        if (t + 1 < n_tiles) {
            stage(b ^ 1);
            ok_cur = ok_pend;
            if (t + 2 < n_tiles) {
                const TileIds next = scalar_ids(t + 2, ids_next);
                fetch(t + 2, next.wave);
                ok_pend = next.bits;
                if (t + 3 < n_tiles) ids_next = load_ids(t + 3);
            }
        }
        __syncthreads();
    }

    // normalise and store: lane holds d = 32db + 8i + 4h + jj of its row
    const float lt = l + __shfl_xor(l, 32);
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

template <int D, int G, int BS>
int launch_prefill(const KvSource& kv, void* out, const void* q, int32_t batch,
                   int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                   int32_t max_seqlen_q, float scale, int32_t causal, hipStream_t stream) {
    const int tok_per_wg = kPrefillRows / G;
    const int64_t n_qtiles = (max_seqlen_q + tok_per_wg - 1) / tok_per_wg;
    const int64_t n_groups = static_cast<int64_t>(kv.num_kv_heads) * batch;
    const int64_t padded = (n_groups + kXcds - 1) / kXcds * n_qtiles * kXcds;
    if (padded > INT32_MAX) return PA_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<uint32_t>(padded));
    hipLaunchKernelGGL((prefill_kernel<D, G, BS>), grid, dim3(kPrefillThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const char*>(kv.k),
                       static_cast<const char*>(kv.v), cu_q, cu_k, kv.table,
                       static_cast<uint16_t*>(out), num_heads, kv.num_kv_heads,
                       kv.num_blocks, kv.max_blocks, scale * kLog2e, causal,
                       static_cast<int32_t>(n_qtiles), static_cast<int32_t>(n_groups));
    return launch_status();
}

template <int D>
int dispatch_prefill_group(int G, const KvSource& kv, void* out, const void* q, int32_t batch,
                           int32_t num_heads, const int32_t* cu_q, const int32_t* cu_k,
                           int32_t max_seqlen_q, float scale, int32_t causal,
                           hipStream_t stream) {
#define PA_PREFILL_LAUNCH(GG, BB) \
    launch_prefill<D, GG, BB>(kv, out, q, batch, num_heads, cu_q, cu_k, max_seqlen_q, scale, causal, stream)
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
                 int32_t max_seqlen_q, float scale, int32_t causal, hipStream_t s) {
    if (num_heads % kv.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || scale == INFINITY) return PA_ERR_INVALID_ARG;
    const int G = num_heads / kv.num_kv_heads;
    if (head_dim == 128)
        return dispatch_prefill_group<128>(G, kv, out, q, batch, num_heads, cu_q, cu_k,
                                           max_seqlen_q, scale, causal != 0, s);
    if (head_dim == 64)
        return dispatch_prefill_group<64>(G, kv, out, q, batch, num_heads, cu_q, cu_k,
                                          max_seqlen_q, scale, causal != 0, s);
    return PA_ERR_UNSUPPORTED;
}

}  // namespace pa

extern "C" int pa_prefill_varlen(const pa_kv_pool* pool, void* out, const void* q, int32_t batch,
                                 int32_t num_heads, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, float softmax_scale, int32_t causal,
                                 void* stream) {
    using namespace pa;
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
    (void)max_seqlen_k;  // the per-request lengths bound the key loop
    // a table of width 0 (possibly null) assigns no block: every row outputs zeros, and
    // the kernel reads no table entry because no request then has a key to load
    const KvSource kv{true, pool->k_cache, pool->v_cache, pool->num_kv_heads, pool->num_blocks,
                      pool->block_size, block_table, max_blocks_per_seq};
    return prefill_impl(kv, pool->head_dim, out, q, batch, num_heads, cu_seqlens_q, cu_seqlens_k,
                        max_seqlen_q, softmax_scale, causal, static_cast<hipStream_t>(stream));
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
