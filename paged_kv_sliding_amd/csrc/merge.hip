// merge.hip -- pairwise merge of two attention partials (v, s) over disjoint
// key sets, the combine sglang's _safe_merge_state dispatches.
//
//   s = ln(exp(s_a) + exp(s_b)),  v = exp(s_a - s) v_a + exp(s_b - s) v_b
//
// The grid runs over (token, head) units, one wavefront each, so the head
// count never enters the block shape (the failure mode the same sglang
// function works around: a block of head_dim/vec x num_heads threads exceeds
// the per-block thread limit for large head counts).
#include <type_traits>

#include "device_common.h"
#include "pkvs_internal.h"

namespace pkvs {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T *p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, int64_t i)
{
    return bf16_bits_to_float(p[i]);
}

template <>
__device__ __forceinline__ float ld<_Float16>(const _Float16 *p, int64_t i)
{
    return float(p[i]);
}

template <typename T>
__device__ __forceinline__ void st(T *p, int64_t i, float x);
template <>
__device__ __forceinline__ void st<float>(float *p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t *p, int64_t i, float x)
{
    p[i] = __builtin_bit_cast(uint16_t, __bf16(x));
}

template <>
__device__ __forceinline__ void st<_Float16>(_Float16 *p, int64_t i, float x)
{
    p[i] = _Float16(x);
}

template <typename T>
__global__ __launch_bounds__(kMergeThreads) void merge_state_kernel(
    const T *va, const float *sa, const T *vb, const float *sb, T *vo, float *so, int64_t units,
    int head_dim)
{
    const int lane = threadIdx.x;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const float a = sa[u], b = sb[u];
        const float M = fmaxf(a, b);
        float wa = 0.f, wb = 0.f, s = kNegInf;
        if (M != kNegInf) {
            constexpr float kLog2e = 1.44269504088896340736f;
            const float ea = fast_exp2((a - M) * kLog2e), eb = fast_exp2((b - M) * kLog2e);
            const float sum = ea + eb;
            s = M + fast_log2(sum) * kLn2;
            wa = ea / sum;
            wb = eb / sum;
        }
        const int64_t base = u * head_dim;
        for (int d = lane; d < head_dim; d += 64) {
            const float x = (wa != 0.f ? wa * ld(va, base + d) : 0.f) +
                            (wb != 0.f ? wb * ld(vb, base + d) : 0.f);
            st(vo, base + d, x);
        }
        if (lane == 0) so[u] = s;
    }
}

// The same combine with 16 bytes of v per lane (8 16-bit or 4 fp32 elements):
// lane c of the grid-stride loop takes 16-byte chunk c of the flattened
// [units, head_dim] arrays, chunk c belongs to unit c >> log2_cpu.  The host
// picks this kernel only when a unit is a power-of-two number of chunks, at
// most 64, so every unit lies within one wave: all its lanes read s_a / s_b
// before its first lane stores s, which keeps in-place use (s_out = s_a) safe.
template <typename T>
__device__ __forceinline__ void widen16(u32x4 x, float (&f)[16 / sizeof(T)])
{
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(x[j]);
    } else if constexpr (std::is_same<T, _Float16>::value) {
        const f32x8 v = __builtin_convertvector(__builtin_bit_cast(f16x8, x), f32x8);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = v[j];
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(x[j] << 16);
            f[2 * j + 1] = __uint_as_float(x[j] & 0xffff0000u);
        }
    }
}

template <typename T>
__device__ __forceinline__ u32x4 narrow16(const float (&f)[16 / sizeof(T)])
{
    if constexpr (sizeof(T) == 4) {
        u32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __float_as_uint(f[j]);
        return x;
    } else {
        f32x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = f[j];
        return __builtin_bit_cast(u32x4, to16x8<std::is_same<T, _Float16>::value>(v));
    }
}

template <typename T>
__global__ __launch_bounds__(kMergeVecThreads) void merge_state_vec_kernel(
    const u32x4 *va, const float *sa, const u32x4 *vb, const float *sb, u32x4 *vo, float *so,
    int64_t chunks, int log2_cpu)
{
    constexpr int E = 16 / sizeof(T);
    constexpr float kLog2e = 1.44269504088896340736f;
    const int64_t stride = int64_t(gridDim.x) * kMergeVecThreads;
    for (int64_t c = int64_t(blockIdx.x) * kMergeVecThreads + threadIdx.x; c < chunks;
         c += stride) {
        const int64_t u = c >> log2_cpu;
        const float a = sa[u], b = sb[u];
        const u32x4 xa = __builtin_nontemporal_load(va + c);
        const u32x4 xb = __builtin_nontemporal_load(vb + c);
        const float M = fmaxf(a, b);
        float wa = 0.f, wb = 0.f, s = kNegInf;
        if (M != kNegInf) {
            const float ea = fast_exp2((a - M) * kLog2e), eb = fast_exp2((b - M) * kLog2e);
            const float sum = ea + eb;
            s = M + fast_log2(sum) * kLn2;
            wa = ea / sum;
            wb = eb / sum;
        }
        float fa[E], fb[E], fo[E];
        widen16<T>(xa, fa);
        widen16<T>(xb, fb);
        // (a partial with weight 0 contributes nothing, whatever its v holds)
#pragma unroll
        for (int j = 0; j < E; ++j)
            fo[j] = (wa != 0.f ? wa * fa[j] : 0.f) + (wb != 0.f ? wb * fb[j] : 0.f);
        __builtin_nontemporal_store(narrow16<T>(fo), vo + c);
        if ((c & ((int64_t(1) << log2_cpu) - 1)) == 0) so[u] = s;
    }
}

}  // namespace

int merge_state_vec_chunks(int32_t head_dim, int32_t dtype)
{
    const int bytes = head_dim * (dtype == PKVS_FP32 ? 4 : 2);
    if (bytes % 16) return 0;
    const int cpu = bytes / 16;
    return (cpu & (cpu - 1)) == 0 && cpu <= 64 ? cpu : 0;
}

hipError_t launch_merge_state_vec(const void *va, const float *sa, const void *vb,
                                  const float *sb, void *vo, float *so, int64_t n, int32_t heads,
                                  int32_t head_dim, int32_t dtype, int grid, hipStream_t s)
{
    const int cpu = merge_state_vec_chunks(head_dim, dtype);
    const int64_t chunks = n * heads * cpu;
    if (chunks == 0) return hipSuccess;
    int log2_cpu = 0;
    while ((1 << log2_cpu) < cpu) ++log2_cpu;
    const auto *a = static_cast<const u32x4 *>(va);
    const auto *b = static_cast<const u32x4 *>(vb);
    auto *o = static_cast<u32x4 *>(vo);
    if (dtype == PKVS_FP16)
        merge_state_vec_kernel<_Float16><<<grid, kMergeVecThreads, 0, s>>>(a, sa, b, sb, o, so,
                                                                          chunks, log2_cpu);
    else if (dtype == PKVS_BF16)
        merge_state_vec_kernel<uint16_t><<<grid, kMergeVecThreads, 0, s>>>(a, sa, b, sb, o, so,
                                                                          chunks, log2_cpu);
    else
        merge_state_vec_kernel<float><<<grid, kMergeVecThreads, 0, s>>>(a, sa, b, sb, o, so,
                                                                       chunks, log2_cpu);
    return hipGetLastError();
}

hipError_t launch_merge_state(const void *va, const float *sa, const void *vb, const float *sb,
                              void *vo, float *so, int64_t n, int32_t heads, int32_t head_dim,
                              int32_t dtype, int grid, hipStream_t s)
{
    const int64_t units = n * heads;
    if (units == 0) return hipSuccess;
    if (dtype == PKVS_FP16)
        merge_state_kernel<_Float16><<<grid, kMergeThreads, 0, s>>>(
            static_cast<const _Float16 *>(va), sa, static_cast<const _Float16 *>(vb), sb,
            static_cast<_Float16 *>(vo), so, units, head_dim);
    else if (dtype == PKVS_BF16)
        merge_state_kernel<uint16_t><<<grid, kMergeThreads, 0, s>>>(
            static_cast<const uint16_t *>(va), sa, static_cast<const uint16_t *>(vb), sb,
            static_cast<uint16_t *>(vo), so, units, head_dim);
    else
        merge_state_kernel<float><<<grid, kMergeThreads, 0, s>>>(
            static_cast<const float *>(va), sa, static_cast<const float *>(vb), sb,
            static_cast<float *>(vo), so, units, head_dim);
    return hipGetLastError();
}

}  // namespace pkvs
