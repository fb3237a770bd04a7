// merge.hip -- pairwise merge of two attention partials (v, s) over disjoint
// key sets, the combine sglang's _safe_merge_state dispatches.
//
//   s = ln(exp(s_a) + exp(s_b)),  v = exp(s_a - s) v_a + exp(s_b - s) v_b
//
// The grid runs over (token, head) units, one wavefront each, so the head
// count never enters the block shape (the failure mode the same sglang
// function works around: a block of head_dim/vec x num_heads threads exceeds
// the per-block thread limit for large head counts).
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

}  // namespace

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
