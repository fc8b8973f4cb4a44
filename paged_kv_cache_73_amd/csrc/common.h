// Internal helpers shared by libpa's HIP sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---- storage types ---------------------------------------------------------------
// bf16 is carried as its raw 16-bit pattern; widening to fp32 places it in the upper
// half of a binary32, which is exact.
struct bf16_t { uint16_t bits; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer descriptor on CDNA (32-bit data format, no swizzle).  A raw
// buffer load whose offset is at or past the descriptor's byte count returns zeros.
constexpr int32_t kBufferDword3 = 0x00020000;

__device__ __forceinline__ uint4 to_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <typename T> struct Storage;
template <> struct Storage<float> { static constexpr int kBytes = 4; };
template <> struct Storage<bf16_t> { static constexpr int kBytes = 2; };

// 16 bytes -> 4 (fp32) or 8 (bf16) floats.
__device__ __forceinline__ void widen(const uint4& w, float (&f)[4], float) {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ void widen(const uint4& w, float (&f)[8], bf16_t) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}

// fp32 -> bf16, round to nearest even (C semantics of the __bf16 conversion; gfx950
// has a native instruction for it).
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

// 4 or 8 floats -> 16 bytes of storage.
__device__ __forceinline__ uint4 narrow(const float (&f)[4], float) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
}
__device__ __forceinline__ uint4 narrow(const float (&f)[8], bf16_t) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        u[i] = static_cast<uint32_t>(to_bf16_bits(f[2 * i])) |
               (static_cast<uint32_t>(to_bf16_bits(f[2 * i + 1])) << 16);
    return make_uint4(u[0], u[1], u[2], u[3]);
}

// ---- cross-lane sums inside groups of LANES consecutive lanes ----------------------
// DPP row permutations: quad_perm [1,0,3,2] and [2,3,0,1] pair lanes at distance 1 and
// 2; after them every lane of a quad holds the quad's sum, so row_half_mirror (lane i
// <-> 7-i of each 8) and row_mirror (i <-> 15-i of each 16) each pair a lane with one
// from the other half and double the group.  Beyond 16 lanes DPP rows end; a
// ds_bpermute shuffle takes over.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LANES == 1 || LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16 ||
                      LANES == 32 || LANES == 64, "group size");
    if constexpr (LANES >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (LANES >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (LANES >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
    if constexpr (LANES >= 16) x += dpp_mov<0x140>(x); // row_mirror
    if constexpr (LANES >= 32) x += __shfl_xor(x, 16);
    if constexpr (LANES >= 64) x += __shfl_xor(x, 32);
    return x;
}

// The two passes of a split-K attention call: partial states (and the rows finished in
// one piece), then their merge.
constexpr int kPass1 = 1, kPass2 = 2;

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

inline int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_BF16 ? 2 : 0); }

inline int check_pool(const pa_kv_pool* pool) {
    if (pool == nullptr || pool->k_cache == nullptr || pool->v_cache == nullptr)
        return PA_ERR_INVALID_ARG;
    if (pool->num_blocks < 0 || pool->block_size <= 0 || pool->num_kv_heads <= 0 ||
        pool->head_dim <= 0)
        return PA_ERR_INVALID_ARG;
    if (elem_bytes(pool->dtype) == 0) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

}  // namespace pa
