// Host side of libpa: reference-counted block manager, metadata builders and
// validators.  No device memory is touched here.
//
// Block manager semantics follow "Paged attention 与 online softmax" §11.3 (reference
// counts, free stack, copy-on-write before writing a shared block) and the worked
// examples of "结合nanovllm的FlashAttention和PagedAttention主要原理概述" 题目4 (blocks
// allocated on demand as a request grows) and 题目6 (free blocks handed out 0,1,2,...;
// deallocation walks the table in reverse; a freed block is the next one reused).

#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_bm {
    std::vector<int32_t> refs;   // reference count per physical block
    std::vector<int32_t> stack;  // free ids; back() is handed out next
    // prefix cache ("结合nanovllm..." 题目6): hash_to_block_id, and per registered block its
    // hash and the token ids it holds (compared on a hit)
    std::unordered_map<uint64_t, int32_t> index;
    std::vector<uint64_t> hash;
    std::vector<uint8_t> hashed;
    std::vector<std::vector<int32_t>> tokens;
};

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

// FNV-1a, 64-bit: for each byte, xor it in, then multiply by the FNV prime.
uint64_t fnv1a(uint64_t h, const uint8_t* p, size_t n) {
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= kFnvPrime;
    }
    return h;
}

// Unregister a block from the prefix cache (freed, or about to be modified).
void forget(pa_bm* bm, int32_t b) {
    if (!bm->hashed[b]) return;
    bm->index.erase(bm->hash[b]);
    bm->hashed[b] = 0;
    bm->tokens[b].clear();
}

}  // namespace

extern "C" {

const char* pa_status_str(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
        case PA_ERR_REFCOUNT: return "PA_ERR_REFCOUNT";
        case PA_ERR_METADATA: return "PA_ERR_METADATA";
        default: return "PA_ERR_UNKNOWN";
    }
}

int32_t pa_abi_version(void) { return 1; }

#ifndef PA_SOURCE_DIGEST
#define PA_SOURCE_DIGEST "unknown"
#endif
const char* pa_source_digest(void) { return PA_SOURCE_DIGEST; }

int pa_bm_create(int32_t num_blocks, const int32_t* initial_order, pa_bm** out) {
    if (out == nullptr || num_blocks < 0) return PA_ERR_INVALID_ARG;
    *out = nullptr;
    pa_bm* bm = new (std::nothrow) pa_bm;
    if (bm == nullptr) return PA_ERR_INVALID_ARG;
    bm->refs.assign(num_blocks, 0);
    bm->stack.resize(num_blocks);
    bm->hash.assign(num_blocks, 0);
    bm->hashed.assign(num_blocks, 0);
    bm->tokens.resize(num_blocks);
    if (initial_order != nullptr) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            const int32_t id = initial_order[i];
            if (id < 0 || id >= num_blocks || seen[id]) {
                delete bm;
                return PA_ERR_INVALID_ARG;
            }
            seen[id] = 1;
        }
    }
    // the first id in hand-out order sits at the top (back) of the stack
    for (int32_t i = 0; i < num_blocks; ++i)
        bm->stack[num_blocks - 1 - i] = initial_order ? initial_order[i] : i;
    *out = bm;
    return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int32_t pa_bm_num_free(const pa_bm* bm) {
    return bm ? static_cast<int32_t>(bm->stack.size()) : 0;
}

int pa_bm_refcount(const pa_bm* bm, int32_t block) {
    if (bm == nullptr || block < 0 || block >= static_cast<int32_t>(bm->refs.size()))
        return PA_ERR_INVALID_ARG;
    return bm->refs[block];
}

int pa_bm_free_stack(const pa_bm* bm, int32_t* out, int32_t capacity, int32_t* count) {
    if (bm == nullptr || count == nullptr || (capacity > 0 && out == nullptr))
        return PA_ERR_INVALID_ARG;
    const int32_t n = static_cast<int32_t>(bm->stack.size());
    *count = n;
    if (capacity < n) return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) out[i] = bm->stack[n - 1 - i];
    return PA_OK;
}

int pa_bm_alloc(pa_bm* bm, int32_t n, int32_t* ids_out) {
    if (bm == nullptr || n < 0 || (n > 0 && ids_out == nullptr)) return PA_ERR_INVALID_ARG;
    if (static_cast<size_t>(n) > bm->stack.size()) return PA_ERR_OUT_OF_BLOCKS;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = bm->stack.back();
        bm->stack.pop_back();
        bm->refs[id] = 1;
        ids_out[i] = id;
    }
    return PA_OK;
}

static bool valid_id(const pa_bm* bm, int32_t block) {
    return block >= 0 && block < static_cast<int32_t>(bm->refs.size());
}

int pa_bm_incref(pa_bm* bm, int32_t block) {
    if (bm == nullptr || !valid_id(bm, block)) return PA_ERR_INVALID_ARG;
    if (bm->refs[block] <= 0) return PA_ERR_REFCOUNT;  // sharing a free block
    ++bm->refs[block];
    return PA_OK;
}

int pa_bm_decref(pa_bm* bm, int32_t block) {
    if (bm == nullptr || !valid_id(bm, block)) return PA_ERR_INVALID_ARG;
    if (bm->refs[block] <= 0) return PA_ERR_REFCOUNT;  // double free
    if (--bm->refs[block] == 0) {
        forget(bm, block);  // a freed block leaves hash_to_block_id (题目6, step 4)
        bm->stack.push_back(block);
    }
    return PA_OK;
}

int pa_bm_release_table(pa_bm* bm, const int32_t* row, int32_t width) {
    if (bm == nullptr || width < 0 || (width > 0 && row == nullptr)) return PA_ERR_INVALID_ARG;
    // check first so that a bad row leaves the manager unchanged
    for (int32_t j = 0; j < width; ++j) {
        if (row[j] < 0) continue;
        if (!valid_id(bm, row[j])) return PA_ERR_INVALID_ARG;
    }
    std::vector<int32_t> drops(bm->refs.size(), 0);
    for (int32_t j = 0; j < width; ++j)
        if (row[j] >= 0 && ++drops[row[j]] > bm->refs[row[j]]) return PA_ERR_REFCOUNT;
    for (int32_t j = width - 1; j >= 0; --j)
        if (row[j] >= 0) pa_bm_decref(bm, row[j]);
    return PA_OK;
}

int pa_bm_share(pa_bm* bm, const int32_t* row, int32_t width, int32_t* row_out) {
    if (bm == nullptr || width < 0 || (width > 0 && (row == nullptr || row_out == nullptr)))
        return PA_ERR_INVALID_ARG;
    for (int32_t j = 0; j < width; ++j) {
        if (row[j] < 0) continue;
        if (!valid_id(bm, row[j])) return PA_ERR_INVALID_ARG;
        if (bm->refs[row[j]] <= 0) return PA_ERR_REFCOUNT;
    }
    for (int32_t j = 0; j < width; ++j) {
        row_out[j] = row[j];
        if (row[j] >= 0) ++bm->refs[row[j]];
    }
    return PA_OK;
}

int pa_bm_prepare_write(pa_bm* bm, int32_t block_size, int32_t* row, int32_t width,
                        int32_t start, int32_t count, int32_t* cow_src, int32_t* cow_dst,
                        int32_t cow_capacity, int32_t* num_cow) {
    if (bm == nullptr || row == nullptr || num_cow == nullptr || block_size <= 0 ||
        width < 0 || start < 0 || count < 0 || cow_capacity < 0)
        return PA_ERR_INVALID_ARG;
    *num_cow = 0;
    if (count == 0) return PA_OK;
    const int64_t last_pos = static_cast<int64_t>(start) + count - 1;
    const int32_t first = start / block_size;
    const int64_t last = last_pos / block_size;
    if (last >= width) return PA_ERR_INVALID_ARG;
    int32_t need = 0, copies = 0;
    for (int32_t lb = first; lb <= last; ++lb) {
        const int32_t id = row[lb];
        if (id < 0) {
            ++need;
        } else {
            if (!valid_id(bm, id) || bm->refs[id] <= 0) return PA_ERR_INVALID_ARG;
            if (bm->refs[id] > 1) ++need, ++copies;
        }
    }
    if (copies > 0 && (cow_src == nullptr || cow_dst == nullptr || copies > cow_capacity))
        return PA_ERR_INVALID_ARG;
    if (static_cast<size_t>(need) > bm->stack.size()) return PA_ERR_OUT_OF_BLOCKS;
    int32_t k = 0;
    for (int32_t lb = first; lb <= last; ++lb) {
        const int32_t old = row[lb];
        if (old < 0) {
            pa_bm_alloc(bm, 1, &row[lb]);
        } else if (bm->refs[old] > 1) {
            int32_t fresh;
            pa_bm_alloc(bm, 1, &fresh);
            pa_bm_decref(bm, old);  // still > 0: another holder keeps it
            row[lb] = fresh;
            cow_src[k] = old;
            cow_dst[k] = fresh;
            ++k;
        } else {
            forget(bm, old);  // a private block about to change no longer matches its hash
        }
    }
    *num_cow = k;
    return PA_OK;
}

uint64_t pa_prefix_block_hash(const int32_t* tokens, int32_t n, uint64_t prefix_hash) {
    uint8_t buf[8];
    for (int i = 0; i < 8; ++i) buf[i] = static_cast<uint8_t>(prefix_hash >> (8 * i));
    uint64_t h = fnv1a(kFnvOffset, buf, 8);
    for (int32_t t = 0; t < n; ++t) {
        const uint32_t u = static_cast<uint32_t>(tokens[t]);
        for (int i = 0; i < 4; ++i) buf[i] = static_cast<uint8_t>(u >> (8 * i));
        h = fnv1a(h, buf, 4);
    }
    return h;
}

int pa_bm_allocate_prefix(pa_bm* bm, int32_t block_size, const int32_t* tokens, int32_t n_tokens,
                          int32_t* row, int32_t width, int32_t* n_hits) {
    if (bm == nullptr || row == nullptr || block_size <= 0 || n_tokens < 0 || width < 0 ||
        (n_tokens > 0 && tokens == nullptr))
        return PA_ERR_INVALID_ARG;
    const int32_t n_full = n_tokens / block_size;
    const int32_t n_blocks = (n_tokens + block_size - 1) / block_size;
    if (n_blocks > width) return PA_ERR_INVALID_ARG;
    // plan first (all or nothing): the chained hash of every full block and its hit
    std::vector<uint64_t> hs(n_full);
    std::vector<int32_t> hit(n_full, -1);
    uint64_t h = 0;
    int32_t misses = n_blocks - n_full;
    for (int32_t i = 0; i < n_full; ++i) {
        const int32_t* chunk = tokens + static_cast<int64_t>(i) * block_size;
        h = pa_prefix_block_hash(chunk, block_size, h);
        hs[i] = h;
        auto it = bm->index.find(h);
        if (it != bm->index.end() &&
            bm->tokens[it->second].size() == static_cast<size_t>(block_size) &&
            std::equal(chunk, chunk + block_size, bm->tokens[it->second].begin()))
            hit[i] = it->second;
        else
            ++misses;
    }
    if (static_cast<size_t>(misses) > bm->stack.size()) return PA_ERR_OUT_OF_BLOCKS;
    int32_t hits = 0;
    for (int32_t j = 0; j < width; ++j) row[j] = -1;
    for (int32_t i = 0; i < n_full; ++i) {
        if (hit[i] >= 0) {
            ++bm->refs[hit[i]];
            row[i] = hit[i];
            ++hits;
            continue;
        }
        int32_t b;
        pa_bm_alloc(bm, 1, &b);
        auto it = bm->index.find(hs[i]);
        if (it != bm->index.end()) forget(bm, it->second);  // collision: the newer block takes the hash
        bm->index[hs[i]] = b;
        bm->hash[b] = hs[i];
        bm->hashed[b] = 1;
        const int32_t* chunk = tokens + static_cast<int64_t>(i) * block_size;
        bm->tokens[b].assign(chunk, chunk + block_size);
        row[i] = b;
    }
    if (n_blocks > n_full) pa_bm_alloc(bm, 1, &row[n_full]);
    if (n_hits) *n_hits = hits;
    return PA_OK;
}

int pa_build_slot_mapping(const int32_t* table, int32_t width, int32_t block_size,
                          const int32_t* seq, const int32_t* pos, int32_t n,
                          int32_t* slots_out) {
    if (n < 0 || width < 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
    if (n > 0 && (table == nullptr || seq == nullptr || pos == nullptr || slots_out == nullptr))
        return PA_ERR_INVALID_ARG;
    // slots are int32: a block whose slots lie past INT32_MAX cannot be named by one, and
    // is refused (before any output is written) rather than wrapped
    for (int32_t i = 0; i < n; ++i) {
        if (seq[i] < 0 || pos[i] < 0 || pos[i] / block_size >= width) return PA_ERR_INVALID_ARG;
        const int64_t phys = table[static_cast<int64_t>(seq[i]) * width + pos[i] / block_size];
        if (phys >= 0 && phys * block_size + pos[i] % block_size > INT32_MAX) return PA_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < n; ++i) {
        const int64_t phys = table[static_cast<int64_t>(seq[i]) * width + pos[i] / block_size];
        slots_out[i] = phys >= 0 ? static_cast<int32_t>(phys * block_size + pos[i] % block_size) : -1;
    }
    return PA_OK;
}

int pa_build_cu_seqlens(const int32_t* lengths, int32_t batch, int32_t* cu_out,
                        int32_t* max_out) {
    if (batch < 0 || cu_out == nullptr || (batch > 0 && lengths == nullptr))
        return PA_ERR_INVALID_ARG;
    int64_t acc = 0;
    int32_t mx = 0;
    for (int32_t i = 0; i < batch; ++i) {
        if (lengths[i] < 0) return PA_ERR_INVALID_ARG;
        acc += lengths[i];
        if (acc > INT32_MAX) return PA_ERR_INVALID_ARG;
    }
    acc = 0;
    cu_out[0] = 0;
    for (int32_t i = 0; i < batch; ++i) {
        acc += lengths[i];
        cu_out[i + 1] = static_cast<int32_t>(acc);
        mx = std::max(mx, lengths[i]);
    }
    if (max_out) *max_out = mx;
    return PA_OK;
}

int64_t pa_pool_bytes(int32_t num_blocks, int32_t block_size, int32_t kv_dim,
                      int32_t elem_bytes) {
    if (num_blocks < 0 || block_size < 0 || kv_dim < 0 || elem_bytes < 0) return PA_ERR_INVALID_ARG;
    return static_cast<int64_t>(num_blocks) * block_size * 2 * kv_dim * elem_bytes;
}

static int check_row(const int32_t* row, int32_t keys, int32_t num_blocks, int32_t block_size) {
    const int32_t used = (keys + block_size - 1) / block_size;
    for (int32_t j = 0; j < used; ++j)
        if (row[j] < 0 || row[j] >= num_blocks) return PA_ERR_METADATA;
    return PA_OK;
}

int pa_validate_decode(const int32_t* table, int32_t batch, int32_t width,
                       const int32_t* seqlens, int32_t max_seqlen_k, int32_t num_blocks,
                       int32_t block_size, int32_t* bad_index) {
    if (bad_index) *bad_index = -1;
    if (batch < 0 || width < 0 || block_size <= 0 || num_blocks < 0 ||
        (batch > 0 && (table == nullptr || seqlens == nullptr)))
        return PA_ERR_INVALID_ARG;
    const int64_t cap = static_cast<int64_t>(width) * block_size;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t n = seqlens[b];
        if (n < 0 || n > max_seqlen_k || n > cap ||
            check_row(table + static_cast<int64_t>(b) * width, n, num_blocks, block_size) != PA_OK) {
            if (bad_index) *bad_index = b;
            return PA_ERR_METADATA;
        }
    }
    return PA_OK;
}

int pa_validate_varlen(const int32_t* table, int32_t batch, int32_t width,
                       const int32_t* cu_q, const int32_t* cu_k, int32_t max_seqlen_q,
                       int32_t max_seqlen_k, int32_t num_blocks, int32_t block_size,
                       int32_t* bad_index) {
    if (bad_index) *bad_index = -1;
    if (batch < 0 || width < 0 || block_size <= 0 || num_blocks < 0 || cu_q == nullptr ||
        cu_k == nullptr || (batch > 0 && table == nullptr))
        return PA_ERR_INVALID_ARG;
    if (cu_q[0] != 0 || cu_k[0] != 0) {
        if (bad_index) *bad_index = 0;
        return PA_ERR_METADATA;
    }
    const int64_t cap = static_cast<int64_t>(width) * block_size;
    for (int32_t i = 0; i < batch; ++i) {
        const int64_t ql = static_cast<int64_t>(cu_q[i + 1]) - cu_q[i];
        const int64_t kl = static_cast<int64_t>(cu_k[i + 1]) - cu_k[i];
        if (ql < 0 || kl < 0 || ql > max_seqlen_q || kl > max_seqlen_k || kl > cap ||
            check_row(table + static_cast<int64_t>(i) * width, static_cast<int32_t>(kl),
                      num_blocks, block_size) != PA_OK) {
            if (bad_index) *bad_index = i;
            return PA_ERR_METADATA;
        }
    }
    return PA_OK;
}

int pa_validate_slots(const int32_t* slots, int32_t n, int32_t num_blocks, int32_t block_size,
                      int32_t* bad_index) {
    if (bad_index) *bad_index = -1;
    if (n < 0 || num_blocks < 0 || block_size <= 0 || (n > 0 && slots == nullptr))
        return PA_ERR_INVALID_ARG;
    const int64_t cap = static_cast<int64_t>(num_blocks) * block_size;
    std::vector<int32_t> seen;
    seen.reserve(n);
    for (int32_t i = 0; i < n; ++i) {
        if (slots[i] < 0) continue;
        if (slots[i] >= cap) {
            if (bad_index) *bad_index = i;
            return PA_ERR_METADATA;
        }
        seen.push_back(slots[i]);
    }
    std::vector<int32_t> sorted = seen;
    std::sort(sorted.begin(), sorted.end());
    auto dup = std::adjacent_find(sorted.begin(), sorted.end());
    if (dup != sorted.end()) {
        for (int32_t i = 0; i < n; ++i)
            if (slots[i] == *dup) {
                // report the second occurrence
                for (int32_t j = i + 1; j < n; ++j)
                    if (slots[j] == *dup) {
                        if (bad_index) *bad_index = j;
                        break;
                    }
                break;
            }
        return PA_ERR_METADATA;
    }
    return PA_OK;
}

}  // extern "C"
