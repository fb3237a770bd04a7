// run.cpp -- run-side entry points of libpkvs: argument checks against the
// plan, kernel launches, and the standalone merge_state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "pkvs_internal.h"
#include "plan_state.h"

using namespace pkvs;

namespace {

// compute units of the current device (256 when it cannot be queried)
int device_cus()
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipGetLastError();
    return cus > 0 ? cus : 256;
}

// Base-2 logit scale and soft-cap factor (see soft_cap_unit): without a cap
// the kernels take exp2(s * sm_scale * log2 e); with a cap c they take
// exp2(c * log2 e * tanh(sm_scale * s / c)).
void logit_scales(const pkvs_desc &d, float sm_scale, float *scale_log2, float *cap_a)
{
    constexpr float kLog2e = 1.44269504088896340736f;
    if (d.logits_soft_cap > 0.f) {
        *scale_log2 = d.logits_soft_cap * kLog2e;
        *cap_a = 2.f * kLog2e * sm_scale / d.logits_soft_cap;
    } else {
        *scale_log2 = sm_scale * kLog2e;
        *cap_a = 0.f;
    }
}

// A k_scale / v_scale must be positive and finite (bit test: the library is
// built with -fno-honor-nans).
bool bad_scale(float x)
{
    uint32_t b;
    std::memcpy(&b, &x, sizeof b);
    return (b >> 31) || (b & 0x7f800000u) == 0x7f800000u || (b & 0x7fffffffu) == 0;
}

int log2_exact(int x)
{
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// The kernels move rows of q, o and the caches in 16-byte vectors.
bool misaligned16(std::initializer_list<const void *> ptrs)
{
    uintptr_t bits = 0;
    for (const void *x : ptrs) bits |= reinterpret_cast<uintptr_t>(x);
    return (bits & 15) != 0;
}

// run() must repeat the window and causality the plan was made for: a run-time
// window that silently replaces the planned one is the mismatch sglang PR
// "Pass window_left at plan time for the SWA paged prefill wrapper" fixes.
int check_run(const pkvs_plan *p, int kind, const void *q, const void *k, const void *v,
              int64_t num_pages, const int32_t *kv_indices, const void *o, int32_t window_left,
              int32_t causal)
{
    if (!p) return fail(PKVS_ERR_INVALID_ARG, "plan is null");
    if (p->desc.kind != kind)
        return fail(PKVS_ERR_INVALID_ARG, kind == PKVS_PREFILL ? "not a prefill plan"
                                                              : "not a decode plan");
    if (window_left != p->desc.window_left)
        return fail(PKVS_ERR_PLAN_MISMATCH, "run window_left %d differs from the planned %d",
                    window_left, p->desc.window_left);
    if (kind == PKVS_PREFILL && causal != p->desc.causal)
        return fail(PKVS_ERR_PLAN_MISMATCH, "run causal %d differs from the planned %d", causal,
                    p->desc.causal);
    if (misaligned16({q, k, v, o}))
        return fail(PKVS_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
    if (!p->planned_device)
        return fail(PKVS_ERR_NOT_PLANNED, "no device plan (plan() failed, was dry, or never "
                    "ran)");
    if (p->n_items > 0 && (!q || !k || !v || !kv_indices || !o || num_pages <= 0))
        return fail(PKVS_ERR_INVALID_ARG, "null tensor or num_pages <= 0");
    return PKVS_OK;
}

// Launch the kernel of a planned prefill pass.  An empty work list still
// launches: the kernels read the item count from the workspace, so a captured
// graph replays correctly after any later plan of the same capacities.  A
// ragged pass reads its keys through the row-index table in front of its
// work list.  With fold_lse set the pass stores the merge of its result with
// the partial (fold_o, fold_lse) of the same queries.
hipError_t launch_prefill_pass(const pkvs_plan *p, const void *q, const void *k, const void *v,
                               int64_t num_pages, const int32_t *kv_indices, void *o, float *lse,
                               float sm_scale, float k_scale, float v_scale, hipStream_t stream,
                               const void *fold_o = nullptr, const float *fold_lse = nullptr,
                               const void *k_ext = nullptr, const void *v_ext = nullptr)
{
    int32_t *ws = static_cast<int32_t *>(p->int_ws);
    PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.kv_indices = p->ragged ? ws : kv_indices;
    a.o = o;
    a.lse = lse;
    a.ws = ws + p->lead_words;
    a.num_pages = p->ragged ? p->desc.qo_capacity : num_pages;
    logit_scales(p->desc, sm_scale * k_scale, &a.scale_log2, &a.cap_a);
    a.v_scale = v_scale;
    a.num_qo_heads = p->desc.num_qo_heads;
    a.num_kv_heads = p->desc.num_kv_heads;
    a.log2_group = log2_exact(p->desc.num_qo_heads / p->desc.num_kv_heads);
    a.page_size = p->desc.page_size;
    a.log2_page = log2_exact(p->desc.page_size);
    a.page_rows = p->ragged ? 1 : p->desc.page_size;
    a.window_left = p->desc.window_left;
    a.causal = p->desc.causal;
    a.fold_o = fold_o;
    a.fold_lse = fold_lse;
    a.table_pages = p->table_pages;
    a.k_ext = k_ext;
    a.v_ext = v_ext;
    if (p->slots_cap > 0) {
        // [slots, group, head_dim] 16-bit, then [slots, group] fp32
        const int group = p->desc.num_qo_heads / p->desc.num_kv_heads;
        a.part_o = p->float_ws;
        a.part_lse = reinterpret_cast<float *>(static_cast<uint16_t *>(p->float_ws) +
                                               p->slots_cap * group * p->desc.head_dim);
    }
    return p->desc.dtype == PKVS_FP32
               ? launch_attention_fp32(a, p->desc.head_dim, p->grid_blocks, stream)
               : launch_prefill_16bit(a, p->desc.head_dim, p->prefill_variant,
                                      p->desc.dtype == PKVS_FP16, p->desc.kv_format,
                                      p->grid_blocks, stream);
}

// The merge of a key-split prefill's chunk partials (decode_merge_kernel: one
// wave per (query token, head), the token's chunks in consecutive slots).  As
// for decode, it is launched under stream capture whenever the plan can split
// (the kernel reads the merge count from the workspace), with a grid fixed by
// the capacities; an eager run of a batch that split nothing skips it.
int launch_key_split_merge(const pkvs_plan *p, void *o, float *lse, hipStream_t stream)
{
    if (p->merges_cap == 0) return PKVS_OK;
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (p->n_merges == 0 && hipStreamIsCapturing(stream, &capture) != hipSuccess)
        return fail(PKVS_ERR_HIP, "hipStreamIsCapturing failed");
    if (p->n_merges == 0 && capture == hipStreamCaptureStatusNone) return PKVS_OK;
    const int group = p->desc.num_qo_heads / p->desc.num_kv_heads;
    DecodeArgs a{};
    a.o = o;
    a.lse = lse;
    a.ws = static_cast<int32_t *>(p->int_ws) + p->lead_words;
    a.part_o16 = static_cast<const uint16_t *>(p->float_ws);
    a.part_lse = reinterpret_cast<float *>(static_cast<uint16_t *>(p->float_ws) +
                                           p->slots_cap * group * p->desc.head_dim);
    a.num_qo_heads = p->desc.num_qo_heads;
    a.num_kv_heads = p->desc.num_kv_heads;
    a.log2_group = log2_exact(group);
    const int grid = int(std::min<int64_t>(
        (p->merges_cap * group + kMergeUnitsPerWave - 1) / kMergeUnitsPerWave, int64_t(p->num_cus) * 64));
    hipError_t e = launch_decode_merge(a, p->desc.head_dim, p->desc.dtype == PKVS_FP16, true,
                                       std::max(grid, 1), stream);
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "key-split merge launch: %s",
                                     hipGetErrorString(e));
    return PKVS_OK;
}

}  // namespace

extern "C" {

int pkvs_prefill_run(const pkvs_plan *p, const void *q, const void *k_cache, const void *v_cache,
                     int64_t num_pages, const int32_t *kv_indices_d, void *o, float *lse,
                     float sm_scale, int32_t window_left, int32_t causal, float k_scale,
                     float v_scale, hipStream_t stream)
{
    clear_error();
    if (bad_scale(k_scale) || bad_scale(v_scale))
        return fail(PKVS_ERR_INVALID_ARG, "k_scale %g / v_scale %g must be positive and finite",
                    double(k_scale), double(v_scale));
    int rc = check_run(p, PKVS_PREFILL, q, k_cache, v_cache, num_pages, kv_indices_d, o,
                       window_left, causal);
    if (rc) return rc;
    hipError_t e = launch_prefill_pass(p, q, k_cache, v_cache, num_pages, kv_indices_d, o, lse,
                                       sm_scale, k_scale, v_scale, stream);
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
    return launch_key_split_merge(p, o, lse, stream);
}

int pkvs_cascade_run(const pkvs_plan *p, const void *q, const void *k_extend,
                     const void *v_extend, const void *k_cache, const void *v_cache,
                     int64_t num_pages, const int32_t *kv_indices_d, void *o, float *lse,
                     float sm_scale, int32_t window_left, float k_scale, float v_scale,
                     hipStream_t stream)
{
    clear_error();
    if (!p) return fail(PKVS_ERR_INVALID_ARG, "plan is null");
    if (p->desc.kind != PKVS_CASCADE) return fail(PKVS_ERR_INVALID_ARG, "not a cascade plan");
    if (bad_scale(k_scale) || bad_scale(v_scale))
        return fail(PKVS_ERR_INVALID_ARG, "k_scale %g / v_scale %g must be positive and finite",
                    double(k_scale), double(v_scale));
    if (window_left != p->desc.window_left)
        return fail(PKVS_ERR_PLAN_MISMATCH, "run window_left %d differs from the planned %d",
                    window_left, p->desc.window_left);
    if (misaligned16({q, k_extend, v_extend, k_cache, v_cache, o}))
        return fail(PKVS_ERR_INVALID_ARG, "q, k_extend, v_extend, k_cache, v_cache and o must "
                    "be 16-byte aligned");
    if (!p->planned_device)
        return fail(PKVS_ERR_NOT_PLANNED, "no device plan (plan() failed, was dry, or never "
                    "ran)");
    if (p->n_items > 0 && (!q || !k_extend || !v_extend || !o))
        return fail(PKVS_ERR_INVALID_ARG, "null q, extend K/V or o");
    if (p->planned_keys > 0 && (!k_cache || !v_cache || !kv_indices_d || num_pages <= 0))
        return fail(PKVS_ERR_INVALID_ARG, "the planned batch has cached keys: null cache, page "
                    "table or num_pages <= 0");
    if (p->fused) {
        // one pass: cached keys from the pages, new keys from k_extend / v_extend
        hipError_t e = launch_prefill_pass(p->pre, q, k_cache, v_cache,
                                           std::max<int64_t>(num_pages, 1), kv_indices_d, o, lse,
                                           sm_scale, k_scale, v_scale, stream, nullptr, nullptr,
                                           k_extend, v_extend);
        if (e != hipSuccess) return fail(PKVS_ERR_HIP, "cascade launch: %s", hipGetErrorString(e));
        return launch_key_split_merge(p->pre, o, lse, stream);
    }
    char *fws = static_cast<char *>(p->float_ws);
    void *o2 = fws + p->o2_off;
    float *lse2 = reinterpret_cast<float *>(fws + p->lse2_off);
    // prefix pass -> (o2, lse2); the extend pass stores the merge of its own
    // (o, lse) with them
    hipError_t e = launch_prefill_pass(p->pre, q, k_cache, v_cache, std::max<int64_t>(num_pages, 1),
                                       kv_indices_d, o2, lse2, sm_scale, k_scale, v_scale, stream);
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "prefix pass launch: %s", hipGetErrorString(e));
    e = launch_prefill_pass(p->ext, q, k_extend, v_extend, 0, nullptr, o, lse, sm_scale, 1.f, 1.f,
                            stream, o2, lse2);
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "extend pass launch: %s", hipGetErrorString(e));
    return PKVS_OK;
}

int pkvs_decode_run(const pkvs_plan *p, const void *q, const void *k_cache, const void *v_cache,
                    int64_t num_pages, const int32_t *kv_indices_d, void *o, float *lse,
                    float sm_scale, int32_t window_left, float k_scale, float v_scale,
                    hipStream_t stream)
{
    clear_error();
    if (bad_scale(k_scale) || bad_scale(v_scale))
        return fail(PKVS_ERR_INVALID_ARG, "k_scale %g / v_scale %g must be positive and finite",
                    double(k_scale), double(v_scale));
    int rc = check_run(p, PKVS_DECODE, q, k_cache, v_cache, num_pages, kv_indices_d, o,
                       window_left, 1);
    if (rc) return rc;
    // (an empty work list still launches: the kernels read the item count
    // from the workspace, so a captured graph replays correctly after any
    // later plan of the same capacities)
    const int log2g = log2_exact(p->desc.num_qo_heads / p->desc.num_kv_heads);
    float scale_log2, cap_a;
    logit_scales(p->desc, sm_scale * k_scale, &scale_log2, &cap_a);
    hipError_t e;
    if (p->desc.dtype == PKVS_FP32) {
        PrefillArgs a{};
        a.q = q;
        a.k = k_cache;
        a.v = v_cache;
        a.kv_indices = kv_indices_d;
        a.o = o;
        a.lse = lse;
        a.ws = static_cast<int32_t *>(p->int_ws);
        a.num_pages = num_pages;
        a.scale_log2 = scale_log2;
        a.cap_a = cap_a;
        a.v_scale = v_scale;
        a.num_qo_heads = p->desc.num_qo_heads;
        a.num_kv_heads = p->desc.num_kv_heads;
        a.log2_group = log2g;
        a.page_size = p->desc.page_size;
        a.log2_page = log2_exact(p->desc.page_size);
        a.page_rows = p->desc.page_size;
        a.window_left = p->desc.window_left;
        a.causal = 1;
        e = launch_attention_fp32(a, p->desc.head_dim, p->grid_blocks, stream);
        if (e != hipSuccess) return fail(PKVS_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
        return PKVS_OK;
    }
    DecodeArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.kv_indices = kv_indices_d;
    a.o = o;
    a.lse = lse;
    a.ws = static_cast<int32_t *>(p->int_ws);
    const int group = p->desc.num_qo_heads / p->desc.num_kv_heads;
    a.part_o = static_cast<float *>(p->float_ws);
    a.part_lse = a.part_o ? a.part_o + p->slots_cap * group * p->desc.head_dim : nullptr;
    a.num_pages = num_pages;
    a.scale_log2 = scale_log2;
    a.cap_a = cap_a;
    a.v_scale = v_scale;
    a.num_qo_heads = p->desc.num_qo_heads;
    a.num_kv_heads = p->desc.num_kv_heads;
    a.log2_group = log2g;
    a.page_size = p->desc.page_size;
    a.log2_page = log2_exact(p->desc.page_size);
    const bool f16 = p->desc.dtype == PKVS_FP16;
    e = launch_decode_16bit(a, p->desc.head_dim, f16, p->desc.kv_format, p->decode_waves,
                            p->grid_blocks, stream);
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    // The merge of split requests' chunk partials.  Under stream capture it is
    // launched whenever the plan can have merges (the kernel reads their
    // count), with a fixed grid sized from the capacity, never from this
    // batch, so a captured graph stays valid for every later plan; an eager
    // run whose planned batch split no request skips it.
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (p->merges_cap > 0 && p->n_merges == 0 &&
        hipStreamIsCapturing(stream, &capture) != hipSuccess)
        return fail(PKVS_ERR_HIP, "hipStreamIsCapturing failed");
    if (p->merges_cap > 0 && (p->n_merges > 0 || capture != hipStreamCaptureStatusNone)) {
        const int grid = int(std::min<int64_t>(
        (p->merges_cap * group + kMergeUnitsPerWave - 1) / kMergeUnitsPerWave, int64_t(p->num_cus) * 64));
        e = launch_decode_merge(a, p->desc.head_dim, f16, false, std::max(grid, 1), stream);
        if (e != hipSuccess)
            return fail(PKVS_ERR_HIP, "decode merge launch: %s", hipGetErrorString(e));
    }
    return PKVS_OK;
}

int pkvs_decode_noalloc(pkvs_plan *p, const int32_t *kv_indptr_h,
                        const int32_t *kv_last_page_len_h, int32_t batch_size, const void *q,
                        const void *k_cache, const void *v_cache, int64_t num_pages,
                        const int32_t *kv_indices_d, void *o, float *lse, float sm_scale,
                        int32_t window_left, float k_scale, float v_scale, hipStream_t stream)
{
    clear_error();
    if (!p) return fail(PKVS_ERR_INVALID_ARG, "plan is null");
    if (p->desc.kind != PKVS_DECODE) return fail(PKVS_ERR_INVALID_ARG, "not a decode plan");
    if (p->desc.dtype == PKVS_FP32)
        return fail(PKVS_ERR_INVALID_ARG, "the allocation-free decode takes bf16 or fp16 plans");
    // the int workspace at the array's start, the float one at the next
    // 256-byte boundary
    const size_t float_off = (p->int_ws_need + 255) / 256 * 256;
    const size_t need = float_off + p->float_ws_need;
    if (need > PKVS_NOALLOC_SCRATCH_BYTES)
        return fail(PKVS_ERR_WORKSPACE, "the plan's workspaces take %zu bytes, more than the "
                    "%zu of the library's scratch array; plan and run with caller workspaces",
                    need, size_t(PKVS_NOALLOC_SCRATCH_BYTES));
    if (!p->have_gpu) return fail(PKVS_ERR_HIP, "no HIP device");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKVS_ERR_HIP, "hipGetDevice failed");
    }
    if (dev != p->device)
        return fail(PKVS_ERR_INVALID_ARG, "the plan was made on device %d but device %d is "
                    "current", p->device, dev);
    void *base = nullptr;
    hipError_t e = scratch_for_device(dev, &base);
    if (e != hipSuccess)
        return fail(PKVS_ERR_HIP, "scratch array of device %d: %s", dev, hipGetErrorString(e));
    char *ws = static_cast<char *>(base);
    int rc = pkvs_decode_plan(p, kv_indptr_h, kv_last_page_len_h, batch_size,
                              p->float_ws_need ? ws + float_off : nullptr, p->float_ws_need, ws,
                              p->int_ws_need, stream);
    if (rc) return rc;
    return pkvs_decode_run(p, q, k_cache, v_cache, num_pages, kv_indices_d, o, lse, sm_scale,
                           window_left, k_scale, v_scale, stream);
}

int pkvs_merge_state(const void *v_a, const float *s_a, const void *v_b, const float *s_b,
                     void *v_out, float *s_out, int64_t num_tokens, int32_t num_heads,
                     int32_t head_dim, int32_t v_dtype, hipStream_t stream)
{
    clear_error();
    if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0)
        return fail(PKVS_ERR_INVALID_ARG, "bad shape (%lld, %d, %d)", (long long)num_tokens,
                    num_heads, head_dim);
    if (v_dtype != PKVS_BF16 && v_dtype != PKVS_FP32 && v_dtype != PKVS_FP16)
        return fail(PKVS_ERR_UNSUPPORTED, "v_dtype %d not built", v_dtype);
    if (num_tokens == 0) return PKVS_OK;
    if (!v_a || !s_a || !v_b || !s_b || !v_out || !s_out)
        return fail(PKVS_ERR_INVALID_ARG, "null pointer");
    const int64_t units = num_tokens * num_heads;
    hipError_t e;
    const int cpu = merge_state_vec_chunks(head_dim, v_dtype);
    const bool aligned = (reinterpret_cast<uintptr_t>(v_a) | reinterpret_cast<uintptr_t>(v_b) |
                          reinterpret_cast<uintptr_t>(v_out)) % 16 == 0;
    if (cpu > 0 && aligned) {
        // 16 bytes per lane; about eight resident workgroups per CU keep
        // enough loads in flight to stream at the HBM rate
        const int64_t chunks = units * cpu;
        const int grid = int(std::min<int64_t>((chunks + kMergeVecThreads - 1) / kMergeVecThreads,
                                               int64_t(device_cus()) * 8));
        e = launch_merge_state_vec(v_a, s_a, v_b, s_b, v_out, s_out, num_tokens, num_heads,
                                   head_dim, v_dtype, grid, stream);
    } else {
        const int grid = int(std::min<int64_t>(units, int64_t(device_cus()) * 32));
        e = launch_merge_state(v_a, s_a, v_b, s_b, v_out, s_out, num_tokens, num_heads, head_dim,
                               v_dtype, grid, stream);
    }
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "merge_state launch: %s", hipGetErrorString(e));
    return PKVS_OK;
}

int pkvs_append_kv(const void *k_new, const void *v_new, const int64_t *loc_d,
                   int64_t num_tokens, void *k_cache, void *v_cache, int64_t num_slots,
                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype, int32_t kv_format,
                   float k_scale, float v_scale, int32_t *status_d, hipStream_t stream)
{
    clear_error();
    if (num_tokens < 0 || num_slots < 0 || num_kv_heads <= 0 || head_dim <= 0)
        return fail(PKVS_ERR_INVALID_ARG, "bad shape (%lld tokens, %lld slots, %d heads, %d "
                    "dims)", (long long)num_tokens, (long long)num_slots, num_kv_heads,
                    head_dim);
    if (dtype != PKVS_BF16 && dtype != PKVS_FP32 && dtype != PKVS_FP16)
        return fail(PKVS_ERR_UNSUPPORTED, "dtype %d not built (bf16, fp16, fp32)", dtype);
    if (kv_format < PKVS_KV_SAME || kv_format > PKVS_KV_FP8_E5M2)
        return fail(PKVS_ERR_INVALID_ARG, "kv_format %d: must be 0, 1 or 2", kv_format);
    const bool eight = kv_format != PKVS_KV_SAME;
    if (eight && (bad_scale(k_scale) || bad_scale(v_scale)))
        return fail(PKVS_ERR_INVALID_ARG, "k_scale %g / v_scale %g must be positive and finite",
                    double(k_scale), double(v_scale));
    const int64_t row_elems = int64_t(num_kv_heads) * head_dim;
    const int64_t row_bytes = row_elems * (dtype == PKVS_FP32 ? 4 : 2);
    if (row_bytes % 16 || row_elems % 8)
        return fail(PKVS_ERR_UNSUPPORTED, "a cache row (num_kv_heads x head_dim elements) "
                    "must be a multiple of 16 bytes and of 8 elements, got %lld elements",
                    (long long)row_elems);
    if (num_tokens == 0) return PKVS_OK;
    if (!k_new || !v_new || !loc_d || !k_cache || !v_cache)
        return fail(PKVS_ERR_INVALID_ARG, "null pointer");
    for (const void *ptr : {k_new, v_new, static_cast<const void *>(k_cache),
                            static_cast<const void *>(v_cache)})
        if (reinterpret_cast<uintptr_t>(ptr) % 16)
            return fail(PKVS_ERR_INVALID_ARG, "k/v rows and caches must be 16-byte aligned");
    const int grid = int(std::min<int64_t>(num_tokens, int64_t(device_cus()) * 16));
    hipError_t e =
        eight ? launch_append_kv_quant(k_new, v_new, loc_d, num_tokens, row_elems, dtype,
                                       kv_format, k_cache, v_cache, num_slots, k_scale, v_scale,
                                       status_d, grid, stream)
              : launch_append_kv(k_new, v_new, loc_d, num_tokens, row_bytes, k_cache, v_cache,
                                 num_slots, status_d, grid, stream);
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "append launch: %s", hipGetErrorString(e));
    return PKVS_OK;
}

int pkvs_build_kv_indices(const int32_t *page_map_d, int64_t map_rows, int64_t map_cols,
                          const int32_t *slot_d, const int32_t *start_d, const int32_t *len_d,
                          int32_t batch_size, int32_t *kv_indptr_d, int32_t *kv_indices_d,
                          int64_t capacity, int32_t *status_d, hipStream_t stream)
{
    clear_error();
    if (batch_size < 0 || map_rows < 0 || map_cols < 0 || capacity < 0)
        return fail(PKVS_ERR_INVALID_ARG, "negative batch, map shape or capacity");
    if (!kv_indptr_d) return fail(PKVS_ERR_INVALID_ARG, "kv_indptr is null");
    if (batch_size > 0 && (!page_map_d || !slot_d || !len_d || (capacity > 0 && !kv_indices_d)))
        return fail(PKVS_ERR_INVALID_ARG, "null map, slot, length or kv_indices array");
    const int grid = int(std::max<int64_t>(1, std::min<int64_t>(batch_size,
                                                                int64_t(device_cus()) * 8)));
    hipError_t e = launch_build_kv_indices(page_map_d, map_rows, map_cols, slot_d, start_d, len_d,
                                           batch_size, kv_indptr_d, kv_indices_d, capacity,
                                           status_d, grid, stream);
    if (e != hipSuccess)
        return fail(PKVS_ERR_HIP, "page-table build launch: %s", hipGetErrorString(e));
    return PKVS_OK;
}

}  // extern "C"
