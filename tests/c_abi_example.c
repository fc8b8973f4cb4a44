/* A plain C user of libpa, with no Python and no PyTorch.
 *
 * "host": the host block manager and metadata builders on the pages' worked examples;
 *   prints one JSON object for the test to compare with the stored examples.
 * "gpu IN OUT" (built with PA_EXAMPLE_GPU): reads a small fp32 paged-decode problem
 *   from IN, takes device memory from the HIP runtime, runs pa_write_kv and pa_decode
 *   through the C ABI, and writes the output rows to OUT.
 *
 * Built and run by tests/test_c_abi.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pa.h"

#ifdef PA_EXAMPLE_GPU
#include <hip/hip_runtime_api.h>
#endif

#define CHECK(call)                                                                \
    do {                                                                           \
        int st_ = (call);                                                          \
        if (st_ != PA_OK) {                                                        \
            fprintf(stderr, "%s failed: %s\n", #call, pa_status_str(st_));         \
            exit(1);                                                               \
        }                                                                          \
    } while (0)

static void print_array(const char* name, const int32_t* a, int n, const char* end) {
    printf("\"%s\": [", name);
    for (int i = 0; i < n; ++i) printf("%s%d", i ? ", " : "", a[i]);
    printf("]%s\n", end);
}

static int host_part(void) {
    printf("{\n\"abi_version\": %d,\n", pa_abi_version());

    /* block table [3, 1, 5], block size 4: the slot of every token of the 10 */
    int32_t table[3] = {3, 1, 5};
    int32_t seq[10], pos[10], slots[10];
    for (int i = 0; i < 10; ++i) {
        seq[i] = 0;
        pos[i] = i;
    }
    CHECK(pa_build_slot_mapping(table, 3, 4, seq, pos, 10, slots));
    print_array("slots_of_tokens_0_to_9", slots, 10, ",");

    /* varlen metadata of query lengths [10, 3, 1] and key lengths [0, 1, 7] */
    int32_t ql[3] = {10, 3, 1}, kl[3] = {0, 1, 7}, cu_q[4], cu_k[4], max_q, max_k;
    CHECK(pa_build_cu_seqlens(ql, 3, cu_q, &max_q));
    CHECK(pa_build_cu_seqlens(kl, 3, cu_k, &max_k));
    print_array("cu_seqlens_q", cu_q, 4, ",");
    print_array("cu_seqlens_k", cu_k, 4, ",");
    printf("\"max_q\": %d, \"max_k\": %d,\n", max_q, max_k);

    /* block manager: a 6-token request (B 4) takes blocks 0 and 1; a second request
     * shares its table; appending token 6 to the second request copies the shared,
     * partly filled block 1 (copy-on-write); releasing both returns every block */
    pa_bm* bm = NULL;
    CHECK(pa_bm_create(8, NULL, &bm));
    int32_t row_a[4] = {-1, -1, -1, -1}, row_b[4], cow_src[4], cow_dst[4], n_cow = 0;
    CHECK(pa_bm_prepare_write(bm, 4, row_a, 4, 0, 6, cow_src, cow_dst, 4, &n_cow));
    print_array("row_a", row_a, 4, ",");
    CHECK(pa_bm_share(bm, row_a, 4, row_b));
    printf("\"refs_after_share\": [%d, %d],\n", pa_bm_refcount(bm, row_a[0]),
           pa_bm_refcount(bm, row_a[1]));
    CHECK(pa_bm_prepare_write(bm, 4, row_b, 4, 6, 1, cow_src, cow_dst, 4, &n_cow));
    print_array("row_b_after_write", row_b, 4, ",");
    print_array("cow_src", cow_src, n_cow, ",");
    print_array("cow_dst", cow_dst, n_cow, ",");
    printf("\"refs_after_cow\": [%d, %d, %d],\n", pa_bm_refcount(bm, 0), pa_bm_refcount(bm, 1),
           pa_bm_refcount(bm, row_b[1]));
    CHECK(pa_bm_release_table(bm, row_b, 4));
    CHECK(pa_bm_release_table(bm, row_a, 4));
    printf("\"free_after_release\": %d,\n", pa_bm_num_free(bm));
    int32_t too_many[9];
    printf("\"alloc_9_of_8\": \"%s\",\n", pa_status_str(pa_bm_alloc(bm, 9, too_many)));
    pa_bm_destroy(bm);

    /* metadata validation: a table entry past the pool is reported */
    int32_t bad_table[2] = {0, 99}, lens[1] = {6}, bad = -1;
    const int st = pa_validate_decode(bad_table, 1, 2, lens, 6, 8, 4, &bad);
    printf("\"validate_bad_table\": \"%s\", \"bad_index\": %d\n}\n", pa_status_str(st), bad);
    return 0;
}

#ifdef PA_EXAMPLE_GPU
#define HIP_CHECK(call)                                                            \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
            exit(1);                                                               \
        }                                                                          \
    } while (0)

static void* read_all(FILE* f, size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (p == NULL || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "short input\n");
        exit(1);
    }
    return p;
}

static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_CHECK(hipMalloc(&d, bytes ? bytes : 4));
    if (bytes) HIP_CHECK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* IN: int32 header {num_blocks, B, Hkv, d, batch, Hq, max_blocks, n_new, max_seqlen_k},
 * float32 scale, then float32 k_pool, v_pool [num_blocks][B][Hkv][d], q [batch][Hq][d],
 * k_new, v_new [n_new][Hkv][d], then int32 table [batch][max_blocks], seqlens [batch],
 * slots [n_new].  OUT: float32 out [batch][Hq][d]. */
static int gpu_part(const char* in_path, const char* out_path) {
    FILE* f = fopen(in_path, "rb");
    if (f == NULL) return 1;
    int32_t hdr[9];
    float scale;
    if (fread(hdr, 4, 9, f) != 9 || fread(&scale, 4, 1, f) != 1) return 1;
    const int32_t nb = hdr[0], B = hdr[1], hkv = hdr[2], d = hdr[3], batch = hdr[4];
    const int32_t hq = hdr[5], width = hdr[6], n_new = hdr[7], max_k = hdr[8];
    const size_t pool = (size_t)nb * B * hkv * d * 4, qb = (size_t)batch * hq * d * 4;
    const size_t newb = (size_t)n_new * hkv * d * 4;
    void* h_k = read_all(f, pool);
    void* h_v = read_all(f, pool);
    void* h_q = read_all(f, qb);
    void* h_kn = read_all(f, newb);
    void* h_vn = read_all(f, newb);
    void* h_table = read_all(f, (size_t)batch * width * 4);
    void* h_lens = read_all(f, (size_t)batch * 4);
    void* h_slots = read_all(f, (size_t)n_new * 4);
    fclose(f);

    pa_kv_pool p;
    p.dtype = PA_F32;
    p.num_blocks = nb;
    p.block_size = B;
    p.num_kv_heads = hkv;
    p.head_dim = d;
    p.k_cache = to_device(h_k, pool);
    p.v_cache = to_device(h_v, pool);
    void* q = to_device(h_q, qb);
    void* kn = to_device(h_kn, newb);
    void* vn = to_device(h_vn, newb);
    void* table = to_device(h_table, (size_t)batch * width * 4);
    void* lens = to_device(h_lens, (size_t)batch * 4);
    void* slots = to_device(h_slots, (size_t)n_new * 4);
    void* out = NULL;
    HIP_CHECK(hipMalloc(&out, qb));
    const size_t ws_bytes = pa_decode_workspace_bytes(batch, hq, hkv, d, max_k, 0, B);
    void* ws = NULL;
    if (ws_bytes) HIP_CHECK(hipMalloc(&ws, ws_bytes));

    CHECK(pa_write_kv(&p, kn, vn, (const int32_t*)slots, n_new, NULL));
    CHECK(pa_decode(&p, out, q, batch, hq, (const int32_t*)table, width, (const int32_t*)lens,
                    max_k, scale, 0, ws, ws_bytes, NULL));
    HIP_CHECK(hipDeviceSynchronize());

    void* h_out = malloc(qb);
    HIP_CHECK(hipMemcpy(h_out, out, qb, hipMemcpyDeviceToHost));
    FILE* o = fopen(out_path, "wb");
    if (o == NULL || fwrite(h_out, 1, qb, o) != qb) return 1;
    fclose(o);
    printf("decode ok: %d sequences, %d heads, workspace %zu bytes\n", batch, hq, ws_bytes);
    return 0;
}
#endif

int main(int argc, char** argv) {
    if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_part();
#ifdef PA_EXAMPLE_GPU
    if (argc == 4 && strcmp(argv[1], "gpu") == 0) return gpu_part(argv[2], argv[3]);
#endif
    fprintf(stderr, "usage: %s host | gpu IN OUT\n", argv[0]);
    return 2;
}
