// plan_state.h -- the opaque pkvs_plan object (host side only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/pkvs.h"

namespace pkvs {

constexpr int kStages = 4;             // pinned staging buffers for the work-list copy
constexpr int kDefaultCus = 256;       // compute units assumed when no device is visible
constexpr int64_t kMinAutoSplit = 256; // smallest key chunk the planner picks by itself
// Decode cost model of the automatic split (measured on MI355X): one wave
// streams one item's K/V at about kWaveBytesPerUs, all waves together at about
// kChipBytesPerUs, and splitting costs a merge launch of about kMergeUs.
constexpr double kWaveBytesPerUs = 10.0e3;
constexpr double kChipBytesPerUs = 5.5e6;
constexpr double kMergeUs = 10.0;
// Key-split prefill (prefill variants 1, 2 and 5): a batch with at most one
// query tile per kSplitFillShare resident workgroups may have its tiles' key
// ranges cut into up to kMaxKeyChunks chunks of whole key tiles, each a work
// item of its own, whose partials a merge combines.  It is cut when its
// longest item, in key tiles, exceeds the longest chunk's by more than
// kMergeTiles (the merge launch, in key tiles of the kernel), and never into
// chunks shorter than kMinChunkTiles.  The chunks of a cut batch number at
// most the resident workgroups, which bounds the partial slots whatever the
// capacities.
constexpr int kMaxKeyChunks = 8;
constexpr int64_t kSplitFillShare = 2;
constexpr int64_t kMergeTiles = 3;
constexpr int64_t kMinChunkTiles = 3;
// prefill_variant = 0, head_dim 128, 16-bit K/V, capacities too small to fill
// the device with 256-row tiles: the 64-key kernel (with the key split) when
// an item can span at least this many keys, else the 128-row kernel
constexpr int64_t kBigSplitKeys = 512;
// decode, pkvs_desc.decode_waves = 0: four waves per work item for batches of
// at most one (request, kv head) pair per kFourWavePairShare resident one-wave
// items whose requests can exceed kFourWaveKeys keys after the window trim
constexpr int64_t kFourWaveKeys = 2048;
constexpr int64_t kFourWavePairShare = 32;

int fail(int code, const char *fmt, ...);
void clear_error();

// Host view of one request's layout, validated.
struct Req {
    int64_t qo_begin, qo_len, kv_len, page_base;
    // one-pass cascade: the request's keys from here on are its new tokens
    int64_t split = INT32_MAX;
};

}  // namespace pkvs

struct pkvs_plan {
    pkvs_desc desc{};
    int device = 0;
    bool have_gpu = false;
    int num_cus = 0;
    int grid_blocks = 0, block_threads = 0, query_tile = 0, item_words = 0;
    int prefill_variant = 1;  // 16-bit prefill kernel variant (PrefillVariant), fixed at creation
    int key_chunks_max = 1;   // prefill: most key chunks per query tile (1: never split)
    int table_pages = 0;      // kPrefillDuo: entries of its LDS page table
    int64_t auto_target_items = 0;
    int decode_waves = 1;     // waves per decode work item (1 or 4)
    int64_t items_cap = 0, slots_cap = 0, merges_cap = 0;
    size_t int_ws_need = 0, float_ws_need = 0;

    // Passes of a cascade prefill (internal prefill plans).  A ragged pass
    // reads keys from a contiguous [tokens, kv heads, head_dim] array indexed
    // like the queries; its page table of row indices sits in the lead_words
    // in front of the work-list header.  A queries_after_kv pass places every
    // query after the last key of its request's table (the cached prefix).
    bool ragged = false;
    bool queries_after_kv = false;
    int64_t lead_words = 0;
    int64_t planned_keys = 0;  // keys of all requests in the last plan()

    // A cascade plan (kind PKVS_CASCADE) owns its two passes and splits the
    // caller's workspaces between them -- or, when `fused`, one prefill plan
    // (pre) over each request's cached keys followed by its new tokens.
    pkvs_plan *ext = nullptr, *pre = nullptr;
    bool fused = false;
    size_t pre_int_off = 0;                         // bytes into int_ws
    size_t o2_off = 0, lse2_off = 0;                // bytes into float_ws

    // the last plan() call
    std::vector<int32_t> host_ws;  // header + items + merge entries
    // decode planning buffers, reserved for the capacities when the plan is
    // created, so that planning a decode batch allocates nothing
    std::vector<pkvs::Req> reqs_buf;
    std::vector<int32_t> merge_buf;
    std::vector<int64_t> req_slot;                // per request: its first partial slot
    std::vector<int32_t> req_chunks;              // per request: its key chunks
    std::vector<uint64_t> order_key;              // per (request, chunk): the order key
    std::vector<int32_t> pair_req, pair_chunk;    // per (request, chunk): its indices
    int64_t n_items = 0, n_merges = 0;
    int32_t split_size = 0;
    int32_t batch = 0;
    bool planned_device = false;
    void *int_ws = nullptr;
    void *float_ws = nullptr;

    // pinned staging ring for the host-to-device copy of the work list
    void *stage[pkvs::kStages] = {};
    hipEvent_t stage_ev[pkvs::kStages] = {};
    bool stage_used[pkvs::kStages] = {};
    int stage_next = 0;
};

namespace pkvs {
using Plan = pkvs_plan;
}
