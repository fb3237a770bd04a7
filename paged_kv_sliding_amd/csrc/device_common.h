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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

// 16-bit inputs -- bfloat16, or IEEE half when F16 -- travel through
// registers and LDS as raw 16-bit patterns held in bf16 vectors; only the
// matrix instructions and the conversions from and to fp32 read them as
// numbers.
template <bool F16>
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> 16-bit, round to nearest even
template <bool F16>
__device__ __forceinline__ bf16x8 to16x8(f32x8 v)
{
    if constexpr (F16) return __builtin_bit_cast(bf16x8, __builtin_convertvector(v, f16x8));
    else return __builtin_convertvector(v, bf16x8);
}

template <bool F16>
__device__ __forceinline__ bf16x4 to16x4(f32x4 v)
{
    if constexpr (F16) return __builtin_bit_cast(bf16x4, __builtin_convertvector(v, f16x4));
    else return __builtin_convertvector(v, bf16x4);
}

template <bool F16>
__device__ __forceinline__ bf16x2 to16x2(f32x2 v)
{
    if constexpr (F16) return __builtin_bit_cast(bf16x2, __builtin_convertvector(v, f16x2));
    else return __builtin_convertvector(v, bf16x2);
}

template <bool F16>
__device__ __forceinline__ uint16_t to16(float x)
{
    if constexpr (F16) return __builtin_bit_cast(uint16_t, _Float16(x));
    else return __builtin_bit_cast(uint16_t, __bf16(x));
}

template <bool F16>
__device__ __forceinline__ float from16(uint16_t x)
{
    if constexpr (F16) return float(__builtin_bit_cast(_Float16, x));
    else return float(__builtin_bit_cast(__bf16, x));
}

template <bool F16>
__device__ __forceinline__ f32x4 from16x4(bf16x4 v)
{
    if constexpr (F16) return __builtin_convertvector(__builtin_bit_cast(f16x4, v), f32x4);
    else return __builtin_convertvector(v, f32x4);
}

// Eight OCP 8-bit floats (KVF 1: e4m3, 2: e5m2) packed in two dwords, byte j
// = element j, widened exactly to fp32 and then to the 16-bit type (also
// exact: every e4m3 and e5m2 value is a bf16 and a half).
template <int KVF, bool F16>
__device__ __forceinline__ bf16x8 widen_fp8(u32x2 raw)
{
    f32x8 f;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        f32x2 lo, hi;
        if constexpr (KVF == 1) {
            lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(raw[w]), false);
            hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(raw[w]), true);
        } else {
            lo = __builtin_amdgcn_cvt_pk_f32_bf8(int(raw[w]), false);
            hi = __builtin_amdgcn_cvt_pk_f32_bf8(int(raw[w]), true);
        }
        f[4 * w] = lo[0];
        f[4 * w + 1] = lo[1];
        f[4 * w + 2] = hi[0];
        f[4 * w + 3] = hi[1];
    }
    return to16x8<F16>(f);
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
