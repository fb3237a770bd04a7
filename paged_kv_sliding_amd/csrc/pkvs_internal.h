// pkvs_internal.h -- work-list formats and tile constants shared by the
// host planner (plan.cpp) and the gfx950 kernels (*.hip) of libpkvs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkvs.h"

namespace pkvs {

// ---------------------------------------------------------------- work list
// The int workspace holds a 64-byte header followed by the items, then the
// merge entries.  Kernels read the counts from the header at run time, so the
// launch grid never depends on one batch.
constexpr int kHeaderWords = 16;
enum HeaderField {
    kHdrNumItems = 0,
    kHdrNumMerges = 1,
    kHdrMergeOffset = 2,  // in int32 words from the start of the workspace
    kHdrItemWords = 3,
    // work counters of the kernels that hand out items at run time: the next
    // item past the first grid-stride round (the decode kernel: one counter;
    // the prefill kernel: one per XCD, kXcds words).  plan() uploads them as
    // 0; a launch with a workgroup for every item never touches them, and in
    // one with fewer workgroups each processed item makes exactly one claim,
    // so the claim that draws the last value puts its counter back to 0:
    // every launch (and graph replay) starts from 0
    kHdrNextItem = 4,
};
// XCDs of the device: consecutive workgroups of a launch go to consecutive
// XCDs (each with its own L2), so workgroup b runs on XCD b mod kXcds
constexpr int kXcds = 8;

// Prefill item: one (request, kv head, query tile).
constexpr int kPrefillItemWords = 12;
enum PrefillItem {
    kPiRequest = 0,
    kPiKvHead = 1,
    kPiQBegin = 2,   // global index of the tile's first query token
    kPiQCount = 3,   // query tokens in the tile
    kPiPos0 = 4,     // sequence position of the first query (prefix + offset)
    kPiKvLen = 5,
    kPiPageBase = 6, // kv_indptr[request]
    kPiKvBegin = 7,  // first key processed (window start rounded down to a key tile)
    kPiSplit = 8,    // one-pass cascade: keys from here on are the request's new
                     // tokens, read from the contiguous K/V (key k on row
                     // k + q_begin - pos0); INT32_MAX: every key is in the cache
    kPiKvEnd = 9,    // one past the last key processed (a multiple of the key tile
                     // past kv_begin unless it is the causal end of the queries)
    kPiSlot = 10,    // -1: write o / lse; else the item is one key chunk of a
                     // split query tile and token r of it writes its partial
                     // (o, lse) to slot kPiSlot + r * kPiSlotStride
    kPiSlotStride = 11,
};

// Decode item: one (request, kv head, key chunk).
constexpr int kDecodeItemWords = 8;
enum DecodeItem {
    kDiRequest = 0,
    kDiKvHead = 1,
    kDiTokBegin = 2, // first key of the chunk (multiple of kDecodeBlock)
    kDiTokEnd = 3,   // one past the last key of the chunk
    kDiVisLo = 4,    // first visible key in the chunk (window start)
    kDiPageBase = 5,
    kDiSlot = 6,     // -1: write o/lse directly; else partial slot index
    kDiKvLen = 7,
};

// Merge entry: the chunks of one (request, kv head) to combine -- for a
// key-split prefill, of one (query token, kv head): kMeRequest is then the
// token's row in q / o.  Both are written to o / lse row kMeRequest.
constexpr int kMergeWords = 4;
enum MergeEntry { kMeRequest = 0, kMeKvHead = 1, kMeFirstSlot = 2, kMeNumSlots = 3 };

// ---------------------------------------------------------------- tiles
// bf16 prefill kernel variants (rows = (query token, head) pairs per workgroup)
enum PrefillVariant {
    kPrefillAuto = 0,
    kPrefillRows128 = 1,  // 4 waves x 32 rows
    kPrefillRows256 = 2,  // 8 waves x 32 rows
    kPrefillWide = 3,     // 4 waves x 64 rows, software-pipelined (head_dim <= 128)
    kPrefillDma = 4,      // 8 waves x 32 rows, K/V rows loaded straight into LDS
                          // (head_dim 128; an item's key range spans at most
                          // kPrefillDmaPages pages)
    kPrefillBig = 5,      // as 4 with 64-key steps and 16-byte loads into an
                          // XOR-swizzled unpadded LDS layout (an item's key
                          // range spans at most kPrefillBigPages pages)
    kPrefillDuo = 6,      // as 5 with 4 waves x 32 rows, two workgroups per CU
                          // (K and V in two-tile rings, a page table sized
                          // from the plan)
};
constexpr int kPrefillBigTile = 64;    // keys per step of kPrefillBig
constexpr int kPrefillDmaPages = 2048;
// kPrefillBig's LDS page table: with one workgroup per CU its 32 KiB fit
// beside the K and V rings, and a window of up to about 8000 keys fits at
// page size 1
constexpr int kPrefillBigPages = 8192;
// A contiguous ("ragged") K/V of [tokens, kv heads, head_dim] is addressed like
// a paged cache whose page-table entries are row indices: entry t of a request
// starting at row r0 is r0 + t * kRaggedPage, and key j sits on row
// entry(j / kRaggedPage) + j % kRaggedPage.
constexpr int kRaggedPage = 256;
constexpr int kPrefillKvTile = 32;     // keys per step
constexpr int kGenericQTile = 16;      // fp32 path: query tokens per item
constexpr int kGenericThreads = 256;
constexpr int kDecodeBlock = 32;       // keys per decode step
constexpr int kDecodeThreads = 64;     // threads per wave of a decode work item
constexpr int kMergeThreads = 64;
// decode_merge_kernel: (merge entry, head) units merged together by one wave
constexpr int kMergeUnitsPerWave = 4;
constexpr int kMergeVecThreads = 256;  // merge_state, 16 bytes of v per lane
constexpr int kAppendThreads = 256;    // cache writes: threads per workgroup (max)
constexpr int kIndptrThreads = 1024;   // page-table build: the running-sum workgroup
constexpr int kGatherThreads = 256;    // page-table build: threads per request

struct PrefillArgs {
    const void *q, *k, *v;
    const int32_t *kv_indices;
    void *o;
    float *lse;
    int32_t *ws;        // int workspace: header (with the work counters) + items
    int64_t num_pages;
    float scale_log2;   // sm_scale * log2(e), or cap * log2(e) with a soft cap
    float cap_a;        // soft cap: 2 log2(e) sm_scale / cap (soft_cap_unit), 0 = none
    float v_scale;      // values are read as v_scale * v (k_scale is in scale_log2 / cap_a)
    int32_t num_qo_heads, num_kv_heads, log2_group, page_size, log2_page;
    int32_t page_rows;  // cache rows one page-table step spans: page_size, or 1 (ragged)
    int32_t window_left, causal;
    // optional partial (o, lse) over other keys of the same queries, laid out
    // like o / lse: when set, the kernel stores the merge of its own result
    // with it (merge_state folded into the epilogue)
    const void *fold_o;
    const float *fold_lse;
    int32_t table_pages;  // kPrefillDuo: entries of its LDS page table (dynamic LDS)
    // one-pass cascade (kPrefillBig): the new tokens' K/V, [tokens, kv heads,
    // head_dim], for the keys at or past each item's kPiSplit; null otherwise
    const void *k_ext, *v_ext;
    // key-split prefill (items with kPiSlot >= 0): partial slots of the float
    // workspace: o in the query dtype (normalised over the chunk's keys), lse
    // in fp32
    void *part_o;     // [slots, group, head_dim]
    float *part_lse;  // [slots, group], natural log
};

struct DecodeArgs {
    const void *q, *k, *v;
    const int32_t *kv_indices;
    void *o;
    float *lse;
    int32_t *ws;      // int workspace: header (with the work counters) + items
    float *part_o;    // [slots, group, head_dim]
    float *part_lse;  // [slots, group]
    // the merge of a key-split prefill: its partial o in the query dtype
    // ([slots, group, head_dim]) instead of part_o
    const uint16_t *part_o16;
    int64_t num_pages;
    float scale_log2;   // as PrefillArgs
    float cap_a;
    float v_scale;
    int32_t num_qo_heads, num_kv_heads, log2_group, page_size, log2_page;
};

// Launchers (return hipError_t of the launch).
// 16-bit paths: bf16, or IEEE half when f16; K/V in the same type (kv_format
// 0) or 8-bit (PKVS_KV_FP8_E4M3 / _E5M2: register-staged prefill variants only)
hipError_t launch_prefill_16bit(const PrefillArgs &a, int head_dim, int variant, bool f16,
                                int kv_format, int grid, hipStream_t s);
hipError_t launch_attention_fp32(const PrefillArgs &a, int head_dim, int grid, hipStream_t s);
// waves: 1 or 4 waves share each decode work item (pkvs_desc.decode_waves)
hipError_t launch_decode_16bit(const DecodeArgs &a, int head_dim, bool f16, int kv_format,
                               int waves, int grid, hipStream_t s);
// p16: the partial o is part_o16, in the query dtype (key-split prefill)
hipError_t launch_decode_merge(const DecodeArgs &a, int head_dim, bool f16, bool p16, int grid,
                               hipStream_t s);
hipError_t launch_merge_state(const void *va, const float *sa, const void *vb, const float *sb,
                              void *vo, float *so, int64_t n, int32_t heads, int32_t head_dim,
                              int32_t dtype, int grid, hipStream_t s);
// 16 bytes per lane: usable when one (token, head) unit of v is a power of two
// of 16-byte chunks, at most 64 (merge_state_vec_chunks > 0) and every v
// pointer is 16-byte aligned; grid in workgroups of kMergeVecThreads
int merge_state_vec_chunks(int32_t head_dim, int32_t dtype);
hipError_t launch_merge_state_vec(const void *va, const float *sa, const void *vb,
                                  const float *sb, void *vo, float *so, int64_t n, int32_t heads,
                                  int32_t head_dim, int32_t dtype, int grid, hipStream_t s);

// Cache writes and page-table build (pool.hip).
hipError_t launch_append_kv(const void *k_new, const void *v_new, const int64_t *loc, int64_t n,
                            int64_t row_bytes, void *k_cache, void *v_cache, int64_t num_slots,
                            int32_t *status, int grid, hipStream_t s);
hipError_t launch_append_kv_quant(const void *k_new, const void *v_new, const int64_t *loc,
                                  int64_t n, int64_t row_elems, int in_dtype, int kv_format,
                                  void *k_cache, void *v_cache, int64_t num_slots, float k_scale,
                                  float v_scale, int32_t *status, int grid, hipStream_t s);
hipError_t launch_build_kv_indices(const int32_t *map, int64_t map_rows, int64_t map_cols,
                                   const int32_t *slot, const int32_t *start, const int32_t *len,
                                   int32_t batch, int32_t *kv_indptr, int32_t *kv_indices,
                                   int64_t capacity, int32_t *status, int grid, hipStream_t s);

// The device address of the library's scratch array on `device` (noalloc.hip),
// which must be the current device at the first call for it; kept per device.
hipError_t scratch_for_device(int device, void **ptr);

// Resident workgroups per CU of each kernel (occupancy query; 0 if unknown).
// (table_pages: the page-table entries of a kPrefillDuo launch)
int prefill_blocks_per_cu(int head_dim, int variant, bool f16, int kv_format,
                          int table_pages = kPrefillDmaPages);
// dynamic LDS bytes of a kPrefillDuo launch with a page table of table_pages entries
size_t prefill_duo_lds_bytes(int table_pages);
int decode_blocks_per_cu(int head_dim, bool f16, int kv_format, int waves);

}  // namespace pkvs
