// pool.hip -- the two steps on either side of the attention kernels: writing
// the batch's new key/value rows into the paged cache, and building the page
// table (kv_indptr, kv_indices) on the device from a request-to-page map.
//
// Both are pure data movement bound by memory traffic: 16-byte vector loads
// and stores, one workgroup per cache row (append) or per request (gather),
// and a single-workgroup running sum for kv_indptr.
#include "device_common.h"
#include "pkvs_internal.h"

namespace pkvs {

namespace {

// Row r of k_new / v_new -> cache slot loc[r] (slot = page * page_size +
// position in the page).  `chunks` = row bytes / 16.  A slot outside the pool
// writes nothing and is counted in status[0].
__global__ __launch_bounds__(kAppendThreads) void append_kv_kernel(
    const u32x4 *__restrict__ k_new, const u32x4 *__restrict__ v_new,
    const int64_t *__restrict__ loc, int64_t n, int chunks, u32x4 *__restrict__ k_cache,
    u32x4 *__restrict__ v_cache, int64_t num_slots, int32_t *status)
{
    for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
        const int64_t s = loc[r];
        if (s < 0 || s >= num_slots) {
            if (status && threadIdx.x == 0) atomicAdd(status, 1);
            continue;
        }
        const u32x4 *kr = k_new + r * chunks, *vr = v_new + r * chunks;
        u32x4 *kd = k_cache + s * chunks, *vd = v_cache + s * chunks;
        for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
            const u32x4 kx = __builtin_nontemporal_load(kr + c);
            const u32x4 vx = __builtin_nontemporal_load(vr + c);
            kd[c] = kx;
            vd[c] = vx;
        }
    }
}

// One element of a new row -> its 8-bit code (KVF 1: e4m3, 2: e5m2), the way
// an 8-bit cache write rounds: the quotient x / scale in fp32 (a correctly
// rounded division), rounded to the input type (IN 0: bf16, 1: fp32, 2: half),
// then to the 8-bit format to nearest even.  Values past the format's range,
// infinities and NaNs get their codes here (e4m3: NaN; e5m2: +-inf, NaN);
// only in-range values go through the hardware's round-to-nearest-even pack.
template <int KVF, int IN>
__device__ __forceinline__ float quant_input(float x, float scale)
{
    float y = x / scale;
    if constexpr (IN == 0) y = float(__bf16(y));
    else if constexpr (IN == 2) y = float(_Float16(y));
    return y;
}

template <int KVF>
__device__ __forceinline__ uint32_t pack_fp8x4(const float (&y)[4])
{
    int w = 0;
    if constexpr (KVF == 1) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], w, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], w, true);
    }
    uint32_t u = uint32_t(w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t b = __float_as_uint(y[i]);
        const uint32_t sign = (b >> 24) & 0x80u;
        const float a = __uint_as_float(b & 0x7fffffffu);
        const bool nan = (b & 0x7fffffffu) > 0x7f800000u;
        uint32_t code = 0xffffffffu;  // keep the packed byte
        if (KVF == 1) {
            if (nan || !(a <= 464.f)) code = sign | 0x7fu;
        } else {
            if (nan) code = sign | 0x7fu;
            else if (!(a < 61440.f)) code = sign | 0x7cu;
        }
        if (code != 0xffffffffu) u = (u & ~(0xffu << (8 * i))) | (code << (8 * i));
    }
    return u;
}

// Rows of k_new / v_new (IN: bf16, fp32 or half; `chunks` = elements / 8 per
// row) quantized into an 8-bit cache at slot loc[r]; out-of-pool slots are
// counted in status[0].
template <int KVF, int IN>
__global__ __launch_bounds__(kAppendThreads) void append_kv_quant_kernel(
    const void *__restrict__ k_new, const void *__restrict__ v_new,
    const int64_t *__restrict__ loc, int64_t n, int chunks, u32x2 *__restrict__ k_cache,
    u32x2 *__restrict__ v_cache, int64_t num_slots, float k_scale, float v_scale, int32_t *status)
{
    for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
        const int64_t s = loc[r];
        if (s < 0 || s >= num_slots) {
            if (status && threadIdx.x == 0) atomicAdd(status, 1);
            continue;
        }
        for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
            const int64_t e0 = (r * chunks + c) * 8;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const void *src = t == 0 ? k_new : v_new;
                const float scale = t == 0 ? k_scale : v_scale;
                float x[8];
                if constexpr (IN == 1) {
                    const f32x4 a = *(static_cast<const f32x4 *>(src) + e0 / 4);
                    const f32x4 b = *(static_cast<const f32x4 *>(src) + e0 / 4 + 1);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = a[i];
                        x[4 + i] = b[i];
                    }
                } else {
                    const u32x4 raw = *(static_cast<const u32x4 *>(src) + e0 / 8);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t w = raw[i];
                        if constexpr (IN == 0) {
                            x[2 * i] = __uint_as_float(w << 16);
                            x[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
                        } else {
                            x[2 * i] = float(__builtin_bit_cast(_Float16, uint16_t(w & 0xffffu)));
                            x[2 * i + 1] = float(__builtin_bit_cast(_Float16, uint16_t(w >> 16)));
                        }
                    }
                }
                float lo[4], hi[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo[i] = quant_input<KVF, IN>(x[i], scale);
                    hi[i] = quant_input<KVF, IN>(x[4 + i], scale);
                }
                const u32x2 out = {pack_fp8x4<KVF>(lo), pack_fp8x4<KVF>(hi)};
                (t == 0 ? k_cache : v_cache)[s * chunks + c] = out;
            }
        }
    }
}

// kv_indptr[0] = 0, kv_indptr[b+1] = kv_indptr[b] + max(len[b], 0), by one
// workgroup: each pass scans kIndptrThreads lengths (wave scans, then the
// wave totals) and carries the total into the next pass.  A negative length
// is counted in status[0].
__global__ __launch_bounds__(kIndptrThreads) void indptr_scan_kernel(
    const int32_t *__restrict__ len, int32_t batch, int32_t *__restrict__ kv_indptr,
    int32_t *status)
{
    constexpr int NW = kIndptrThreads / 64;
    __shared__ int32_t wave_sum[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int32_t carry = 0;
    if (tid == 0) kv_indptr[0] = 0;
    for (int32_t base = 0; base < batch; base += kIndptrThreads) {
        const int32_t b = base + tid;
        int32_t v = 0;
        if (b < batch) {
            v = len[b];
            if (v < 0) {
                if (status) atomicAdd(status, 1);
                v = 0;
            }
        }
        // inclusive scan within the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t u = __shfl_up(v, d);
            if (lane >= d) v += u;
        }
        if (lane == 63) wave_sum[wave] = v;
        __syncthreads();
        int32_t before = carry;
        for (int w = 0; w < wave; ++w) before += wave_sum[w];
        if (b < batch) kv_indptr[b + 1] = before + v;
        int32_t total = 0;
        for (int w = 0; w < NW; ++w) total += wave_sum[w];
        carry += total;
        __syncthreads();  // wave_sum is rewritten by the next pass
    }
}

// kv_indices[kv_indptr[b] + j] = map[slot[b]][start[b] + j] for j < the
// request's length (from kv_indptr).  A source outside the map gives -1; an
// entry at or past `capacity` is not written; each is counted in status[0].
__global__ __launch_bounds__(kGatherThreads) void gather_indices_kernel(
    const int32_t *__restrict__ map, int64_t map_rows, int64_t map_cols,
    const int32_t *__restrict__ slot, const int32_t *__restrict__ start, int32_t batch,
    const int32_t *__restrict__ kv_indptr, int32_t *__restrict__ kv_indices, int64_t capacity,
    int32_t *status)
{
    for (int32_t b = blockIdx.x; b < batch; b += gridDim.x) {
        const int64_t base = kv_indptr[b];
        const int64_t n = int64_t(kv_indptr[b + 1]) - base;
        const int64_t row = slot[b];
        const int64_t s0 = start ? start[b] : 0;
        const bool row_ok = row >= 0 && row < map_rows;
        for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
            const int64_t dst = base + j;
            if (dst >= capacity) {
                if (status) atomicAdd(status, 1);
                continue;
            }
            const int64_t col = s0 + j;
            const bool ok = row_ok && col >= 0 && col < map_cols;
            if (!ok && status) atomicAdd(status, 1);
            kv_indices[dst] = ok ? map[row * map_cols + col] : -1;
        }
    }
}

}  // namespace

hipError_t launch_append_kv(const void *k_new, const void *v_new, const int64_t *loc, int64_t n,
                            int64_t row_bytes, void *k_cache, void *v_cache, int64_t num_slots,
                            int32_t *status, int grid, hipStream_t s)
{
    const int chunks = int(row_bytes / 16);
    const int threads = chunks >= kAppendThreads ? kAppendThreads : (chunks + 63) / 64 * 64;
    append_kv_kernel<<<grid, threads, 0, s>>>(
        static_cast<const u32x4 *>(k_new), static_cast<const u32x4 *>(v_new), loc, n, chunks,
        static_cast<u32x4 *>(k_cache), static_cast<u32x4 *>(v_cache), num_slots, status);
    return hipGetLastError();
}

template <int KVF>
static hipError_t launch_quant_t(const void *k_new, const void *v_new, const int64_t *loc,
                                 int64_t n, int chunks, int in_dtype, void *k_cache,
                                 void *v_cache, int64_t num_slots, float k_scale, float v_scale,
                                 int32_t *status, int grid, int threads, hipStream_t s)
{
    u32x2 *kc = static_cast<u32x2 *>(k_cache), *vc = static_cast<u32x2 *>(v_cache);
    switch (in_dtype) {
    case PKVS_BF16:
        append_kv_quant_kernel<KVF, 0><<<grid, threads, 0, s>>>(
            k_new, v_new, loc, n, chunks, kc, vc, num_slots, k_scale, v_scale, status);
        break;
    case PKVS_FP32:
        append_kv_quant_kernel<KVF, 1><<<grid, threads, 0, s>>>(
            k_new, v_new, loc, n, chunks, kc, vc, num_slots, k_scale, v_scale, status);
        break;
    case PKVS_FP16:
        append_kv_quant_kernel<KVF, 2><<<grid, threads, 0, s>>>(
            k_new, v_new, loc, n, chunks, kc, vc, num_slots, k_scale, v_scale, status);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_append_kv_quant(const void *k_new, const void *v_new, const int64_t *loc,
                                  int64_t n, int64_t row_elems, int in_dtype, int kv_format,
                                  void *k_cache, void *v_cache, int64_t num_slots, float k_scale,
                                  float v_scale, int32_t *status, int grid, hipStream_t s)
{
    const int chunks = int(row_elems / 8);
    const int threads = chunks >= kAppendThreads ? kAppendThreads : (chunks + 63) / 64 * 64;
    return kv_format == PKVS_KV_FP8_E4M3
               ? launch_quant_t<1>(k_new, v_new, loc, n, chunks, in_dtype, k_cache, v_cache,
                                   num_slots, k_scale, v_scale, status, grid, threads, s)
               : launch_quant_t<2>(k_new, v_new, loc, n, chunks, in_dtype, k_cache, v_cache,
                                   num_slots, k_scale, v_scale, status, grid, threads, s);
}

hipError_t launch_build_kv_indices(const int32_t *map, int64_t map_rows, int64_t map_cols,
                                   const int32_t *slot, const int32_t *start, const int32_t *len,
                                   int32_t batch, int32_t *kv_indptr, int32_t *kv_indices,
                                   int64_t capacity, int32_t *status, int grid, hipStream_t s)
{
    indptr_scan_kernel<<<1, kIndptrThreads, 0, s>>>(len, batch, kv_indptr, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || batch == 0) return e;
    gather_indices_kernel<<<grid, kGatherThreads, 0, s>>>(map, map_rows, map_cols, slot, start,
                                                          batch, kv_indptr, kv_indices, capacity,
                                                          status);
    return hipGetLastError();
}

}  // namespace pkvs
