// device_common.h -- small device helpers shared by the libpkvs kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkvs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Logits soft cap: with a = 2 log2(e) * sm_scale / cap, the capped logit
// cap * tanh(sm_scale * s / cap) is cap * soft_cap_unit(s, a), from
// tanh(y) = 1 - 2 / (e^(2y) + 1) (limits exactly -1 and +1 for large |y|).
__device__ __forceinline__ float soft_cap_unit(float s, float a)
{
    const float e = fast_exp2(s * a);
    return 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b)
{
    return __uint_as_float(uint32_t(b) << 16);
}

// Page id of logical key `tok` of a request whose pages start at
// kv_indices[page_base]; clamped into [0, num_pages) so that a corrupt page
// table can never send a load outside the cache.
__device__ __forceinline__ int64_t page_of(const int32_t *__restrict__ kv_indices, int page_base,
                                           int tok, int log2_page, int64_t num_pages)
{
    int64_t pg = kv_indices[page_base + (tok >> log2_page)];
    pg = pg < 0 ? 0 : pg;
    return pg >= num_pages ? num_pages - 1 : pg;
}

// Element offset of (page, slot, kv head, dim 0) in an NHD cache.
__device__ __forceinline__ int64_t nhd_offset(int64_t page, int slot, int page_size, int hk,
                                              int num_kv_heads, int head_dim)
{
    return ((page * page_size + slot) * num_kv_heads + hk) * int64_t(head_dim);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const void *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ bf16x8 zero_bf16x8()
{
    u32x4 z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, z);
}

}  // namespace pkvs
