// plan.cpp -- host side of libpkvs: plan objects, work-list construction,
// workspace sizing, error reporting.
//
// The planner follows the statement of the problem on the pages:
//  * window_left (and causal) are fixed at plan time, and run() must repeat
//    them (sglang PR "Pass window_left at plan time for the SWA paged prefill
//    wrapper", section "What");
//  * the plan is built from host-known CSR arrays, with no device-to-host copy
//    (sglang flashinfer_backend.py, fast_prefill_plan);
//  * decode keeps only the last min(kv_len, W+1) keys of a request
//    (FlashInferIndicesUpdaterDecode.update_sliding_window), and long key
//    ranges are cut into fixed-size chunks whose partial results are merged
//    (fixed_split_size of the deterministic-inference settings);
//  * a prefill query tile starts reading keys at the tile that holds the
//    window start of its first query (the per-tile KV-start skip); the exact
//    mask is still applied per element by the kernels;
//  * the grid and workspaces are sized from capacities and the device only,
//    and a batch beyond the capacity is rejected, never under-launched
//    (AMD-Ecosystem/flashinfer PR 234, "Why each fix" 2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "pkvs_internal.h"
#include "plan_state.h"

namespace pkvs {

static thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

static bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Work-list order key: decreasing cost (0 <= cost < 2^31), then increasing
// index; sorting the keys as plain integers gives that order (std::sort is in
// place: a plan of a reserved size allocates nothing).
static uint64_t sort_key(int64_t cost, int64_t index)
{
    return (uint64_t(uint32_t(INT32_MAX - std::min<int64_t>(cost, INT32_MAX))) << 32) |
           uint32_t(index);
}

// Capacity-derived sizes; depend on the descriptor and the device only.
static void size_plan(Plan *p)
{
    const pkvs_desc &d = p->desc;
    const int64_t B = d.batch_capacity;
    const int64_t hkv = d.num_kv_heads;
    const int64_t group = d.num_qo_heads / d.num_kv_heads;
    int64_t items = 0, slots = 0, merges = 0;
    if (d.kind == PKVS_PREFILL) {
        items = hkv * (ceil_div(d.qo_capacity, p->query_tile) + B);
        if (p->key_chunks_max > 1) {
            // A batch is cut only with at most grid / kSplitFillShare tiles,
            // into at most grid chunks in all (see build_prefill); a tile of n
            // tokens cut into c chunks takes n * c slots and n merge entries.
            const int64_t cut_tiles = p->grid_blocks / kSplitFillShare;
            const int64_t cut_items = p->grid_blocks;
            items = std::max(items, cut_items);
            slots = int64_t(p->query_tile) * cut_items;
            merges = int64_t(p->query_tile) * cut_tiles;
        }
        // a ragged pass's row-index table: at most one entry per kRaggedPage
        // tokens of each request, rounded up per request
        if (p->ragged) p->lead_words = (ceil_div(d.qo_capacity, kRaggedPage) + B + 15) / 16 * 16;
    } else {
        // keys a request can present after the window trim, plus the
        // alignment of the first chunk to a key block
        int64_t nmax = d.kv_capacity;
        if (d.window_left >= 0) nmax = std::min<int64_t>(nmax, int64_t(d.window_left) + 1);
        nmax += kDecodeBlock - 1;
        int64_t per_req;
        if (d.disable_split_kv || d.dtype == PKVS_FP32) {
            per_req = 1;
        } else if (d.fixed_split_size > 0) {
            per_req = std::max<int64_t>(1, ceil_div(nmax, d.fixed_split_size));
        } else {
            // automatic chunking never makes more than B + target/hkv chunks
            // per head in total (see choose_split); bound per request by the
            // smallest automatic chunk
            per_req = std::max<int64_t>(1, ceil_div(nmax, kMinAutoSplit));
        }
        items = B * hkv * per_req;
        if (d.fixed_split_size <= 0 && !d.disable_split_kv && d.dtype != PKVS_FP32)
            items = std::min<int64_t>(items, B * hkv * 2 + int64_t(p->auto_target_items) + hkv);
        items = std::max<int64_t>(items, B * hkv);
        slots = (per_req > 1) ? items : 0;
        merges = (per_req > 1) ? B * hkv : 0;
    }
    p->items_cap = items;
    p->slots_cap = slots;
    p->merges_cap = merges;
    p->int_ws_need = sizeof(int32_t) * size_t(p->lead_words + kHeaderWords +
                                              items * p->item_words + merges * kMergeWords);
    // partial (o, lse) per slot and query head: fp32 o for decode, o in the
    // query dtype for a key-split prefill; fp32 lse
    p->float_ws_need = size_t(slots * group) *
                       (size_t(d.head_dim) * (d.kind == PKVS_PREFILL ? 2 : 4) + sizeof(float));
}

static int validate_desc(const pkvs_desc *d)
{
    if (!d) return fail(PKVS_ERR_INVALID_ARG, "desc is null");
    if (d->kind != PKVS_PREFILL && d->kind != PKVS_DECODE && d->kind != PKVS_CASCADE)
        return fail(PKVS_ERR_INVALID_ARG, "kind must be PKVS_PREFILL, PKVS_DECODE or "
                    "PKVS_CASCADE");
    const bool prefill_like = d->kind != PKVS_DECODE;
    if (d->num_qo_heads <= 0 || d->num_kv_heads <= 0 || d->num_qo_heads % d->num_kv_heads)
        return fail(PKVS_ERR_INVALID_ARG, "num_qo_heads (%d) must be a positive multiple of "
                    "num_kv_heads (%d)", d->num_qo_heads, d->num_kv_heads);
    const int group = d->num_qo_heads / d->num_kv_heads;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
        return fail(PKVS_ERR_UNSUPPORTED, "head_dim %d not built (64, 128, 256)", d->head_dim);
    if (!is_pow2(d->page_size) || d->page_size > 1024)
        return fail(PKVS_ERR_UNSUPPORTED, "page_size %d must be a power of two <= 1024",
                    d->page_size);
    const int64_t page_rows = d->kind == PKVS_CASCADE ? std::max(d->page_size, kRaggedPage)
                                                      : d->page_size;
    if (page_rows * d->num_kv_heads * d->head_dim >= (int64_t(1) << 31))
        return fail(PKVS_ERR_UNSUPPORTED, "one page (page_size x num_kv_heads x head_dim "
                    "elements, %d rows for a cascade's extend keys) must stay below 2^31 "
                    "elements", kRaggedPage);
    if (d->dtype != PKVS_BF16 && d->dtype != PKVS_FP32 && d->dtype != PKVS_FP16)
        return fail(PKVS_ERR_UNSUPPORTED, "dtype %d not built (bf16, fp16, fp32)", d->dtype);
    if (d->dtype != PKVS_FP32 && (!is_pow2(group) || group > 16))
        return fail(PKVS_ERR_UNSUPPORTED, "the 16-bit paths need a power-of-two group <= 16, "
                    "got %d", group);
    // (bit test: this file is built with -fno-honor-nans, which folds NaN
    // comparisons away)
    uint32_t cap_bits;
    std::memcpy(&cap_bits, &d->logits_soft_cap, sizeof cap_bits);
    if ((cap_bits & 0x7f800000u) == 0x7f800000u || ((cap_bits >> 31) && (cap_bits << 1)))
        return fail(PKVS_ERR_INVALID_ARG, "logits_soft_cap %g: must be 0 (off) or a positive "
                    "finite cap", double(d->logits_soft_cap));
    if (d->kv_format < PKVS_KV_SAME || d->kv_format > PKVS_KV_FP8_E5M2)
        return fail(PKVS_ERR_INVALID_ARG, "kv_format %d: must be 0 (same as dtype), 1 (e4m3) or "
                    "2 (e5m2)", d->kv_format);
    if (d->kv_format != PKVS_KV_SAME && d->dtype == PKVS_FP32)
        return fail(PKVS_ERR_UNSUPPORTED, "8-bit K/V are built for bf16 and fp16 queries");
    if (d->kv_format != PKVS_KV_SAME &&
        (d->prefill_variant == kPrefillWide || d->prefill_variant == kPrefillDma ||
         d->prefill_variant == kPrefillBig || d->prefill_variant == kPrefillDuo))
        return fail(PKVS_ERR_UNSUPPORTED, "8-bit K/V are widened on the register-staged prefill "
                    "variants (1, 2)");
    if (d->window_left < -1)
        return fail(PKVS_ERR_INVALID_ARG, "window_left %d: must be -1 (off) or >= 0",
                    d->window_left);
    if (prefill_like && d->causal != 1 && !(d->causal == 0 && d->window_left == -1))
        return fail(PKVS_ERR_UNSUPPORTED, "non-causal prefill is built only without a window");
    if (d->fixed_split_size != -1 && (d->fixed_split_size <= 0 ||
                                      d->fixed_split_size % kDecodeBlock))
        return fail(PKVS_ERR_INVALID_ARG, "fixed_split_size %d must be -1 or a positive "
                    "multiple of %d", d->fixed_split_size, kDecodeBlock);
    if (d->decode_waves != 0 && d->decode_waves != 1 && d->decode_waves != 4)
        return fail(PKVS_ERR_INVALID_ARG, "decode_waves %d must be 0 (planner's choice), 1 or 4",
                    d->decode_waves);
    if (d->prefill_variant < 0 || d->prefill_variant > 6)
        return fail(PKVS_ERR_INVALID_ARG, "prefill_variant %d must be 0..6", d->prefill_variant);
    if (d->prefill_variant > 1 && d->head_dim > 128)
        return fail(PKVS_ERR_UNSUPPORTED, "256-row prefill variants are built for head_dim <= 128");
    if ((d->prefill_variant == kPrefillDma || d->prefill_variant == kPrefillBig ||
         d->prefill_variant == kPrefillDuo) &&
        d->head_dim != 128)
        return fail(PKVS_ERR_UNSUPPORTED, "the direct-to-LDS prefill variants are built for "
                    "head_dim 128");
    if (d->batch_capacity <= 0 || d->kv_capacity <= 0 ||
        (prefill_like && d->qo_capacity <= 0))
        return fail(PKVS_ERR_INVALID_ARG, "capacities must be positive");
    if (d->kv_capacity > (int64_t(1) << 30) || d->qo_capacity > (int64_t(1) << 30))
        return fail(PKVS_ERR_UNSUPPORTED, "capacities above 2^30 tokens are not supported");
    return PKVS_OK;
}

static int read_layout(const Plan *p, const int32_t *qo_indptr, const int32_t *kv_indptr,
                       const int32_t *last, int32_t batch, std::vector<Req> &out)
{
    const pkvs_desc &d = p->desc;
    if (batch < 0) return fail(PKVS_ERR_INVALID_ARG, "batch_size %d < 0", batch);
    if (batch > d.batch_capacity)
        return fail(PKVS_ERR_CAPACITY, "batch_size %d exceeds batch_capacity %d", batch,
                    d.batch_capacity);
    if (!kv_indptr || (batch > 0 && !last) || (d.kind == PKVS_PREFILL && !qo_indptr))
        return fail(PKVS_ERR_INVALID_ARG, "null layout array");
    if (kv_indptr[0] != 0 || (qo_indptr && qo_indptr[0] != 0))
        return fail(PKVS_ERR_INVALID_ARG, "indptr arrays must start at 0");
    out.resize(batch);
    int64_t total_q = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t np = int64_t(kv_indptr[b + 1]) - kv_indptr[b];
        if (np < 0) return fail(PKVS_ERR_INVALID_ARG, "kv_indptr decreases at request %d", b);
        int64_t kv_len = 0;
        if (np > 0) {
            if (last[b] < 1 || last[b] > d.page_size)
                return fail(PKVS_ERR_INVALID_ARG, "kv_last_page_len[%d] = %d outside [1, %d]", b,
                            last[b], d.page_size);
            kv_len = (np - 1) * d.page_size + last[b];
        }
        int64_t qo_len = 1, qo_begin = b;
        if (d.kind == PKVS_PREFILL) {
            qo_begin = qo_indptr[b];
            qo_len = int64_t(qo_indptr[b + 1]) - qo_indptr[b];
            if (qo_len < 0) return fail(PKVS_ERR_INVALID_ARG, "qo_indptr decreases at %d", b);
            if (qo_len > kv_len && !p->queries_after_kv)
                return fail(PKVS_ERR_INVALID_ARG, "request %d: qo_len %lld > kv_len %lld", b,
                            (long long)qo_len, (long long)kv_len);
        }
        if (kv_len > d.kv_capacity)
            return fail(PKVS_ERR_CAPACITY, "request %d: kv_len %lld exceeds kv_capacity %lld", b,
                        (long long)kv_len, (long long)d.kv_capacity);
        total_q += (d.kind == PKVS_PREFILL) ? qo_len : 0;
        out[b] = Req{qo_begin, qo_len, kv_len, kv_indptr[b]};
    }
    if (d.kind == PKVS_PREFILL && total_q > d.qo_capacity)
        return fail(PKVS_ERR_CAPACITY, "total query tokens %lld exceed qo_capacity %lld",
                    (long long)total_q, (long long)d.qo_capacity);
    return PKVS_OK;
}

// Prefill work list: (request, kv head, query tile).  The first key tile of an
// item is the one holding the window start of its first query; the last is
// the one holding its last query's position (causal).  Items are ordered by
// decreasing key count, so the longest start first; the kv heads of one tile
// (equal counts) are consecutive.  The order is a sort of the query tiles (or
// key chunks), not of the items: every kv head of a tile has its key count.
static int build_prefill(Plan *p, const std::vector<Req> &reqs)
{
    const pkvs_desc &d = p->desc;
    const int tq = p->query_tile;
    const int64_t H = d.num_kv_heads;
    const int kv_tile = p->prefill_variant == kPrefillBig || p->prefill_variant == kPrefillDuo
                            ? kPrefillBigTile
                            : kPrefillKvTile;
    // a query tile, or one key chunk of one (all kv heads)
    struct Tile {
        int32_t b, q_begin, qn, pos0, kv_begin, kv_end;
        int32_t slot, chunks;  // first partial slot of kv head 0 (-1: not cut), chunks of the tile
    };
    std::vector<Tile> tiles;
    for (size_t b = 0; b < reqs.size(); ++b) {
        const Req &r = reqs[b];
        // first query position: after the request's cached prefix, or (a
        // cascade's prefix pass) after every key of its table
        const int64_t prefix = p->queries_after_kv ? r.kv_len : r.kv_len - r.qo_len;
        for (int64_t t0 = 0; t0 < r.qo_len; t0 += tq) {
            const int64_t qn = std::min<int64_t>(tq, r.qo_len - t0);
            const int64_t pos0 = prefix + t0;
            int64_t kv_begin = 0;
            if (d.window_left >= 0) kv_begin = std::max<int64_t>(0, pos0 - d.window_left);
            kv_begin = kv_begin / kv_tile * kv_tile;
            const int64_t kv_end = d.causal ? std::min<int64_t>(r.kv_len, pos0 + qn) : r.kv_len;
            tiles.push_back(Tile{int32_t(b), int32_t(r.qo_begin + t0), int32_t(qn), int32_t(pos0),
                                 int32_t(kv_begin), int32_t(std::max(kv_end, kv_begin)), -1, 1});
        }
    }
    auto tiles_of = [&](const Tile &t) { return ceil_div(int64_t(t.kv_end) - t.kv_begin, kv_tile); };
    // Key split: with at most one tile per kSplitFillShare resident
    // workgroups (per kv head), cut the longest tiles' key ranges into chunks
    // of about c whole key tiles (each a work item per kv head with partial
    // slots), c the smallest chunk length with at most one item per resident
    // workgroup in all (a second round would undo the cut), when the longest
    // item then ends sooner by more than the merge costs; the merge entries
    // combine each token's chunks.
    std::vector<int32_t> merges;
    if (p->key_chunks_max > 1 && int64_t(tiles.size()) * H * kSplitFillShare <= p->grid_blocks) {
        int64_t total = 0, longest = 0;
        for (const Tile &t : tiles) {
            total += tiles_of(t) * H;
            longest = std::max(longest, tiles_of(t));
        }
        int64_t c = 0;
        // chunks of a tile of t key tiles for chunk length c (at most
        // key_chunks_max, none empty)
        auto chunks_of = [&](int64_t t) {
            const int64_t n = std::max<int64_t>(1, std::min<int64_t>(p->key_chunks_max, ceil_div(t, c)));
            return t > 0 ? ceil_div(t, ceil_div(t, n)) : int64_t(1);
        };
        auto items_at = [&](int64_t len) {
            c = len;
            int64_t n = 0;
            for (const Tile &t : tiles) n += chunks_of(tiles_of(t)) * H;
            return n;
        };
        // (items_at is non-increasing in the length; at the longest tile it
        // is the uncut count)
        int64_t lo = std::max<int64_t>(kMinChunkTiles, ceil_div(total, p->grid_blocks));
        int64_t hi = std::max(lo, longest);
        while (lo < hi) {
            const int64_t mid = (lo + hi) / 2;
            if (items_at(mid) <= p->grid_blocks) hi = mid;
            else lo = mid + 1;
        }
        items_at(lo);
        int64_t longest_chunk = 0;
        for (const Tile &t : tiles)
            longest_chunk = std::max(longest_chunk, ceil_div(tiles_of(t), chunks_of(tiles_of(t))));
        if (longest > longest_chunk + kMergeTiles) {
            std::vector<Tile> cut;
            int64_t slot = 0;
            for (const Tile &t : tiles) {
                const int64_t kt = tiles_of(t);
                const int64_t n = chunks_of(kt);
                if (n <= 1) {
                    cut.push_back(t);
                    continue;
                }
                // kv head hk's token r, chunk k: slot + (hk qn + r) n + k
                if (slot + H * t.qn * n > p->slots_cap ||
                    int64_t(merges.size() / kMergeWords) + H * t.qn > p->merges_cap)
                    return fail(PKVS_ERR_CAPACITY, "key-split prefill needs more partial slots "
                                "than the plan's %lld", (long long)p->slots_cap);
                for (int64_t hk = 0; hk < H; ++hk)
                    for (int64_t r = 0; r < t.qn; ++r)
                        merges.insert(merges.end(), {int32_t(t.q_begin + r), int32_t(hk),
                                                     int32_t(slot + (hk * t.qn + r) * n),
                                                     int32_t(n)});
                // n chunks of per key tiles, the last one shorter (never empty)
                const int64_t per = ceil_div(kt, n);
                for (int64_t k = 0; k < n; ++k) {
                    Tile ch = t;
                    ch.kv_begin = int32_t(t.kv_begin + k * per * kv_tile);
                    ch.kv_end = k + 1 == n ? t.kv_end : int32_t(ch.kv_begin + per * kv_tile);
                    ch.slot = int32_t(slot + k);
                    ch.chunks = int32_t(n);
                    cut.push_back(ch);
                }
                slot += H * t.qn * n;
            }
            tiles.swap(cut);
        }
    }
    // the direct-to-LDS variants keep an item's page ids in an LDS table; the
    // variant was fixed at plan creation so that no item within the
    // capacities can span more pages than the table (item_pages_bound)
    if (p->prefill_variant == kPrefillDma || p->prefill_variant == kPrefillBig ||
        p->prefill_variant == kPrefillDuo) {
        const int64_t table = p->prefill_variant == kPrefillDuo ? int64_t(p->table_pages)
                              : p->prefill_variant == kPrefillBig ? int64_t(kPrefillBigPages)
                                                                  : int64_t(kPrefillDmaPages);
        for (const Tile &t : tiles) {
            const int64_t kb = t.kv_begin, kv_len = reqs[size_t(t.b)].kv_len;
            if (t.kv_end <= kb) continue;
            const int64_t last = std::min(kb + ceil_div(t.kv_end - kb, kv_tile) * kv_tile,
                                          kv_len) - 1;
            if (last / d.page_size - kb / d.page_size + 1 > table)
                return fail(PKVS_ERR_CAPACITY, "a prefill item spans %lld pages of keys, more "
                            "than the %lld the plan's kernel holds",
                            (long long)(last / d.page_size - kb / d.page_size + 1),
                            (long long)table);
        }
    }
    // longest first, ties in the order made
    std::vector<uint64_t> order(tiles.size());
    for (size_t i = 0; i < tiles.size(); ++i)
        order[i] = sort_key(int64_t(tiles[i].kv_end) - tiles[i].kv_begin, int64_t(i));
    std::sort(order.begin(), order.end());
    const int64_t n_items = int64_t(tiles.size()) * H;
    p->n_items = n_items;
    p->n_merges = int64_t(merges.size() / kMergeWords);
    p->split_size = 0;
    const size_t merge_off = kHeaderWords + size_t(n_items) * kPrefillItemWords;
    p->host_ws.assign(p->lead_words + merge_off + merges.size(), 0);
    int64_t keys = 0;
    for (const Req &r : reqs) keys += r.kv_len;
    p->planned_keys = keys;
    if (p->ragged) {
        // row-index table: entry t of request b is the row of its key
        // t * kRaggedPage in the contiguous K/V (rows follow the queries)
        for (const Req &r : reqs)
            for (int64_t t = 0; t * kRaggedPage < r.kv_len; ++t)
                p->host_ws[r.page_base + t] = int32_t(r.qo_begin + t * kRaggedPage);
    }
    int32_t *w = p->host_ws.data() + p->lead_words;
    w[kHdrNumItems] = int32_t(n_items);
    w[kHdrNumMerges] = int32_t(p->n_merges);
    w[kHdrMergeOffset] = int32_t(merge_off);
    w[kHdrItemWords] = kPrefillItemWords;
    // (ties in the order made: (tile, kv head, chunk) -- each run of
    // equal-length chunks of one tile is emitted kv head by kv head)
    int32_t *it = w + kHeaderWords;
    for (size_t i0 = 0, i1; i0 < order.size(); i0 = i1) {
        const Tile &t0 = tiles[size_t(uint32_t(order[i0]))];
        for (i1 = i0 + 1; i1 < order.size() && (order[i1] >> 32) == (order[i0] >> 32) &&
                          tiles[size_t(uint32_t(order[i1]))].q_begin == t0.q_begin &&
                          tiles[size_t(uint32_t(order[i1]))].b == t0.b;
             ++i1) {
        }
        for (int64_t hk = 0; hk < H; ++hk)
            for (size_t i = i0; i < i1; ++i, it += kPrefillItemWords) {
                const Tile &t = tiles[size_t(uint32_t(order[i]))];
                const Req &r = reqs[size_t(t.b)];
                it[kPiRequest] = t.b;
                it[kPiKvHead] = int32_t(hk);
                it[kPiQBegin] = t.q_begin;
                it[kPiQCount] = t.qn;
                it[kPiPos0] = t.pos0;
                it[kPiKvLen] = int32_t(r.kv_len);
                it[kPiPageBase] = int32_t(r.page_base);
                it[kPiKvBegin] = t.kv_begin;
                it[kPiSplit] = int32_t(std::min<int64_t>(r.split, INT32_MAX));
                it[kPiKvEnd] = t.kv_end;
                it[kPiSlot] = t.slot < 0 ? -1 : int32_t(t.slot + hk * t.qn * t.chunks);
                it[kPiSlotStride] = t.slot < 0 ? 0 : t.chunks;
            }
    }
    std::copy(merges.begin(), merges.end(), w + merge_off);
    return PKVS_OK;
}

// Keys per decode chunk when the caller leaves it to the planner: aim for
// about auto_target_items chunks over the whole batch (one per resident wave)
// so every wave gets work in one round, but never cut below kMinAutoSplit keys,
// and split only when the estimated time of the split batch (its bytes at the
// chip's rate, or its longest chunk at one wave's, plus the merge) beats one
// wave per request and kv head streaming the longest request.
static int64_t choose_split(const Plan *p, const std::vector<Req> &reqs)
{
    const pkvs_desc &d = p->desc;
    int64_t longest = kDecodeBlock, total = 0;
    for (const Req &r : reqs) {
        int64_t ws = d.window_left >= 0 ? std::max<int64_t>(0, r.kv_len - 1 - d.window_left) : 0;
        int64_t n = r.kv_len - ws / kDecodeBlock * kDecodeBlock;
        longest = std::max(longest, n);
        total += n;
    }
    const int64_t no_split = ceil_div(longest, kDecodeBlock) * kDecodeBlock;
    if (d.disable_split_kv || d.dtype == PKVS_FP32) return no_split;
    if (d.fixed_split_size > 0) return d.fixed_split_size;
    const int64_t units = int64_t(reqs.size()) * d.num_kv_heads;
    const int64_t target = p->auto_target_items;
    if (units >= target) return no_split;
    int64_t c = ceil_div(total * d.num_kv_heads, target);
    c = ceil_div(c, kDecodeBlock) * kDecodeBlock;
    c = std::min(no_split, std::max<int64_t>(c, kMinAutoSplit));
    const double key_bytes =
        2.0 * d.head_dim * (d.kv_format != PKVS_KV_SAME ? 1 : 2);  // K and V of one key, one head
    const double item_rate = kWaveBytesPerUs * p->decode_waves;  // one item's streaming rate
    const double t_whole = double(longest) * key_bytes / item_rate;
    const double t_split = std::max(double(total) * d.num_kv_heads * key_bytes / kChipBytesPerUs,
                                    double(c) * key_bytes / item_rate) + kMergeUs;
    return t_whole <= t_split ? no_split : c;
}

static int build_decode(Plan *p, const std::vector<Req> &reqs)
{
    const pkvs_desc &d = p->desc;
    const int64_t c = choose_split(p, reqs);
    const int64_t H = d.num_kv_heads;
    // (the buffers were reserved for the capacities: no allocation here)
    std::vector<int32_t> &merges = p->merge_buf;
    std::vector<int64_t> &first_slot = p->req_slot;  // per request: slot of kv head 0, chunk 0
    std::vector<int32_t> &chunks = p->req_chunks;    // per request: its chunks
    std::vector<uint64_t> &order = p->order_key;     // per (request, chunk): sort_key
    std::vector<int32_t> &pair_req = p->pair_req, &pair_chunk = p->pair_chunk;
    merges.clear();
    first_slot.clear();
    chunks.clear();
    order.clear();
    pair_req.clear();
    pair_chunk.clear();
    int64_t slot = 0, n_items = 0;
    for (size_t b = 0; b < reqs.size(); ++b) {
        const Req &r = reqs[b];
        const int64_t ws =
            d.window_left >= 0 ? std::max<int64_t>(0, r.kv_len - 1 - d.window_left) : 0;
        const int64_t base = ws / kDecodeBlock * kDecodeBlock;
        int64_t nchunks = r.kv_len == 0 ? 1 : ceil_div(r.kv_len - base, c);
        // a trailing piece shorter than one key block joins the chunk before it
        // rather than becoming a work item and a partial of its own
        if (nchunks > 1 && r.kv_len - base - (nchunks - 1) * c < kDecodeBlock) --nchunks;
        if (n_items + H * nchunks > p->items_cap ||
            (nchunks > 1 && (slot + H * nchunks > p->slots_cap ||
                             int64_t(merges.size() / kMergeWords) + H > p->merges_cap)))
            return fail(PKVS_ERR_CAPACITY, "decode work list exceeds the plan capacity (%lld "
                        "items, %lld partial slots) at request %zu", (long long)p->items_cap,
                        (long long)p->slots_cap, b);
        // kv head hk's chunk k of a split request: slot first + hk nchunks + k
        first_slot.push_back(nchunks > 1 ? slot : -1);
        chunks.push_back(int32_t(nchunks));
        if (nchunks > 1) {
            for (int64_t hk = 0; hk < H; ++hk)
                merges.insert(merges.end(), {int32_t(b), int32_t(hk), int32_t(slot + hk * nchunks),
                                             int32_t(nchunks)});
            slot += H * nchunks;
        }
        for (int64_t k = 0; k < nchunks; ++k) {
            const int64_t t0 = base + k * c;
            const int64_t t1 = k + 1 == nchunks ? r.kv_len : t0 + c;
            order.push_back(sort_key(t1 - t0, int64_t(pair_req.size())));
            pair_req.push_back(int32_t(b));
            pair_chunk.push_back(int32_t(k));
        }
        n_items += H * nchunks;
    }
    // longest first, ties in the order made: (request, kv head, chunk) -- the
    // chunks are sorted and each run of equal-length chunks of one request
    // is emitted kv head by kv head.  (Kv heads made consecutive items
    // instead measured 6 % slower on the 64-request decode with no window.)
    std::sort(order.begin(), order.end());
    p->n_items = n_items;
    p->n_merges = int64_t(merges.size() / kMergeWords);
    p->split_size = int32_t(std::min<int64_t>(c, INT32_MAX));
    const size_t merge_off = kHeaderWords + size_t(n_items) * kDecodeItemWords;
    p->host_ws.assign(merge_off + merges.size(), 0);
    int32_t *w = p->host_ws.data();
    w[kHdrNumItems] = int32_t(n_items);
    w[kHdrNumMerges] = int32_t(p->n_merges);
    w[kHdrMergeOffset] = int32_t(merge_off);
    w[kHdrItemWords] = kDecodeItemWords;
    int32_t *it = w + kHeaderWords;
    for (size_t i0 = 0, i1; i0 < order.size(); i0 = i1) {
        const int32_t b = pair_req[size_t(uint32_t(order[i0]))];
        for (i1 = i0 + 1; i1 < order.size() && (order[i1] >> 32) == (order[i0] >> 32) &&
                          pair_req[size_t(uint32_t(order[i1]))] == b;
             ++i1) {
        }
        const Req &r = reqs[size_t(b)];
        const int64_t n = chunks[size_t(b)];
        const int64_t ws =
            d.window_left >= 0 ? std::max<int64_t>(0, r.kv_len - 1 - d.window_left) : 0;
        for (int64_t hk = 0; hk < H; ++hk)
            for (size_t i = i0; i < i1; ++i, it += kDecodeItemWords) {
                const int64_t k = pair_chunk[size_t(uint32_t(order[i]))];
                const int64_t t0 = ws / kDecodeBlock * kDecodeBlock + k * c;
                const int64_t t1 = k + 1 == n ? r.kv_len : t0 + c;
                it[kDiRequest] = b;
                it[kDiKvHead] = int32_t(hk);
                it[kDiTokBegin] = int32_t(t0);
                it[kDiTokEnd] = int32_t(t1);
                it[kDiVisLo] = int32_t(std::max(ws, t0));
                it[kDiPageBase] = int32_t(r.page_base);
                it[kDiSlot] = first_slot[size_t(b)] < 0
                                  ? -1
                                  : int32_t(first_slot[size_t(b)] + hk * n + k);
                it[kDiKvLen] = int32_t(r.kv_len);
            }
    }
    std::copy(merges.begin(), merges.end(), w + merge_off);
    return PKVS_OK;
}

// The pinned staging ring of a plan's work-list copies, made once per plan.
static int make_staging(Plan *p)
{
    if (p->stage[0]) return PKVS_OK;
    for (int i = 0; i < kStages; ++i) {
        if (hipHostMalloc(&p->stage[i], p->int_ws_need, hipHostMallocDefault) != hipSuccess ||
            hipEventCreateWithFlags(&p->stage_ev[i], hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            return fail(PKVS_ERR_HIP, "pinned staging buffer of %zu bytes: allocation failed",
                        p->int_ws_need);
        }
    }
    return PKVS_OK;
}

// Copy the host work list into the device int workspace with one async
// host-to-device copy on `stream`, from a ring of pinned staging buffers (a
// buffer is reused only after its previous copy has completed).
static int upload(Plan *p, void *int_ws, hipStream_t stream)
{
    const size_t bytes = p->host_ws.size() * sizeof(int32_t);
    int rc = make_staging(p);  // (a decode plan made it at creation)
    if (rc) return rc;
    const int s = p->stage_next;
    p->stage_next = (s + 1) % kStages;
    if (p->stage_used[s] && hipEventSynchronize(p->stage_ev[s]) != hipSuccess)
        return fail(PKVS_ERR_HIP, "waiting for a staging buffer failed");
    std::memcpy(p->stage[s], p->host_ws.data(), bytes);
    hipError_t e = hipMemcpyAsync(int_ws, p->stage[s], bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
    e = hipEventRecord(p->stage_ev[s], stream);
    if (e != hipSuccess) return fail(PKVS_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
    p->stage_used[s] = true;
    return PKVS_OK;
}

static int finish_plan(Plan *p, void *float_ws, size_t float_bytes, void *int_ws,
                       size_t int_bytes, hipStream_t stream)
{
    p->planned_device = false;
    if (!int_ws) return PKVS_OK;  // dry plan
    if (int_bytes < p->int_ws_need)
        return fail(PKVS_ERR_WORKSPACE, "int workspace %zu bytes < required %zu; increase the "
                    "workspace buffer size", int_bytes, p->int_ws_need);
    if (p->float_ws_need && (!float_ws || float_bytes < p->float_ws_need))
        return fail(PKVS_ERR_WORKSPACE, "float workspace %zu bytes < required %zu; increase "
                    "the workspace buffer size", float_ws ? float_bytes : 0, p->float_ws_need);
    if ((reinterpret_cast<uintptr_t>(int_ws) | reinterpret_cast<uintptr_t>(float_ws)) & 15)
        return fail(PKVS_ERR_INVALID_ARG, "the workspaces must be 16-byte aligned");
    if (!p->have_gpu) return fail(PKVS_ERR_HIP, "no HIP device: only dry plans are possible");
    int rc = upload(p, int_ws, stream);
    if (rc) return rc;
    p->int_ws = int_ws;
    p->float_ws = float_ws;
    p->planned_device = true;
    return PKVS_OK;
}

// Most pages of keys one prefill item can span within the plan's capacities.
// Its first key tile starts at most kv_tile-1 keys before the window start of
// its first query, and its last (cut at the request's end) ends at most
// kv_tile-2 keys past its last query's position, so with a window the span is
// below window_left + query_tile + 2 kv_tile keys; without one it is at most
// the whole request.  (A cascade's prefix pass places its queries after every
// key of the table, which only shortens the span.)
static int64_t item_pages_bound(const pkvs_desc &d, int kv_tile, int query_tile)
{
    const int64_t P = d.page_size;
    int64_t pages = (d.kv_capacity - 1) / P + 1;
    if (d.window_left >= 0 && d.causal) {
        const int64_t span = int64_t(d.window_left) + query_tile + 2 * int64_t(kv_tile) - 3;
        pages = std::min(pages, span / P + 2);
    }
    return pages;
}

static void destroy_plan(Plan *p);

// A validated prefill or decode descriptor -> plan object (ragged: a
// cascade's extend pass, see plan_state.h).
static int create_plan(const pkvs_desc *desc, bool ragged, Plan **out, bool make_buffers = true,
                       bool key_split = true)
{
    Plan *p = new (std::nothrow) Plan();
    if (!p) return fail(PKVS_ERR_INVALID_ARG, "out of host memory");
    p->desc = *desc;
    p->ragged = ragged;
    const int group = desc->num_qo_heads / desc->num_kv_heads;
    int ndev = 0;
    p->have_gpu = hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0 &&
                  hipGetDevice(&p->device) == hipSuccess;
    p->num_cus = kDefaultCus;
    if (p->have_gpu) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device) ==
                hipSuccess && cus > 0)
            p->num_cus = cus;
    }
    (void)hipGetLastError();
    const bool fp32 = desc->dtype == PKVS_FP32, f16 = desc->dtype == PKVS_FP16;
    const int kvf = desc->kv_format;
    if (desc->kind == PKVS_PREFILL) {
        // Kernel variant: 256-row workgroups (8 waves x 32 rows) share each
        // staged key tile between more rows and keep two waves per SIMD; they
        // are the fastest measured for head_dim <= 128, and for head_dim 128
        // with 16-bit K/V the 64-key-step direct-to-LDS kernel is the fastest
        // of them.  128-row workgroups serve head_dim 256 and batches too small
        // to fill the device with 256-row tiles -- except that with the key
        // split (which fills the device by cutting key ranges) the 64-key
        // kernel is also the faster one for head_dim 128 once an item can
        // span kBigSplitKeys keys (measured: chunks of long prompts, prompts
        // of 1024 tokens and more).  Variants 3 and 4 are available on request.
        const int64_t big_tiles = ceil_div(desc->qo_capacity, 256 / group) * desc->num_kv_heads;
        int v = kPrefillRows128;
        bool big_for_split = false;
        if (desc->head_dim <= 128 && big_tiles >= 2 * p->num_cus) {
            // (below 8 keys per page every lane of the 64-key kernel loads its
            // own row, and with the device full the 256-row kernel measured
            // 1.4 % faster at page size 1)
            v = desc->head_dim == 128 && kvf == PKVS_KV_SAME && desc->page_size >= 8
                    ? kPrefillBig
                    : kPrefillRows256;
        } else if (key_split && !desc->disable_split_kv && !ragged && !fp32 &&
                   desc->head_dim == 128 && kvf == PKVS_KV_SAME) {
            int64_t span = desc->kv_capacity;
            if (desc->window_left >= 0 && desc->causal)
                span = std::min<int64_t>(span, int64_t(desc->window_left) + 256 / group);
            if (span >= kBigSplitKeys) {
                v = kPrefillBig;
                big_for_split = true;
            }
        }
        if (desc->prefill_variant) {
            v = desc->prefill_variant;
            big_for_split = false;
        }
        // the direct-to-LDS variants need 104-156 KiB of LDS per workgroup
        // ... and an LDS table of at most kPrefillDmaPages page ids per item
        // (kPrefillBig: kPrefillBigPages): they are kept only when no item
        // within the capacities can span more pages (kPrefillDuo sizes its
        // table to that span).  The choice holds
        // for the plan's lifetime, so a captured run keeps launching the
        // kernel that every later plan() builds its items for.
        const bool dma_v = v == kPrefillDma || v == kPrefillBig || v == kPrefillDuo;
        int64_t span = 0;
        if (dma_v) {
            span = item_pages_bound(*desc, v == kPrefillDma ? kPrefillKvTile : kPrefillBigTile,
                                    (v == kPrefillDuo ? 128 : 256) / group);
            if (span > (v == kPrefillBig ? kPrefillBigPages : kPrefillDmaPages))
                v = big_for_split ? kPrefillRows128 : kPrefillRows256;
        }
        if (v == kPrefillDuo) p->table_pages = int(std::min<int64_t>(kPrefillDmaPages,
                                                                     (span + 15) / 16 * 16));
        if ((v == kPrefillDma || v == kPrefillBig || v == kPrefillDuo) && p->have_gpu && !fp32 &&
            prefill_blocks_per_cu(desc->head_dim, v, f16, kvf, p->table_pages) < 1)
            v = big_for_split ? kPrefillRows128 : kPrefillRows256;
        p->prefill_variant = v;
        const int rows = v == kPrefillRows128 || v == kPrefillDuo ? 128 : 256;
        p->query_tile = fp32 ? kGenericQTile : rows / group;
        p->item_words = kPrefillItemWords;
        p->block_threads =
            fp32 ? kGenericThreads
                 : (v == kPrefillRows256 || v == kPrefillDma || v == kPrefillBig ? 512 : 256);
        int per_cu = p->have_gpu && !fp32
                         ? prefill_blocks_per_cu(desc->head_dim, v, f16, kvf, p->table_pages)
                         : 0;
        p->grid_blocks = p->num_cus * std::max(per_cu, fp32 ? 2 : 1);
        // Key split on the 128- and 256-row register-staged kernels and the
        // default 64-key one: fixed here, like the partial slots it needs
        // (sized from the grid), so that a captured run stays valid for every
        // plan; plan() cuts only batches of few query tiles.
        if (key_split && !desc->disable_split_kv && !ragged && !fp32 &&
            (v == kPrefillRows128 || v == kPrefillRows256 || v == kPrefillBig))
            p->key_chunks_max = kMaxKeyChunks;
    } else {
        p->query_tile = 1;
        p->item_words = fp32 ? kPrefillItemWords : kDecodeItemWords;
        // Waves per work item: four when the batch has at most one (request,
        // kv head) pair per kFourWavePairShare resident one-wave items (one
        // wave per SIMD when the occupancy cannot be queried) and a request
        // can present more than kFourWaveKeys keys after the window trim.
        // One wave per item would then cut each pair into many short chunks
        // whose merge dominates; four waves per item need a quarter of the
        // chunks and combine within the item in LDS.  For larger batches or
        // shorter requests one wave per item measured as fast or faster.
        const int per_cu1 =
            p->have_gpu && !fp32 ? decode_blocks_per_cu(desc->head_dim, f16, kvf, 1) : 0;
        int nw = desc->decode_waves;
        if (nw == 0) {
            int64_t keys = desc->kv_capacity;
            if (desc->window_left >= 0) keys = std::min<int64_t>(keys, int64_t(desc->window_left) + 1);
            nw = int64_t(desc->batch_capacity) * desc->num_kv_heads * kFourWavePairShare <=
                             int64_t(p->num_cus) * (per_cu1 > 0 ? per_cu1 : 4) &&
                         keys > kFourWaveKeys
                     ? 4
                     : 1;
        }
        if (fp32) nw = 1;
        p->decode_waves = nw;
        p->block_threads = fp32 ? kGenericThreads : kDecodeThreads * nw;
        const int per_cu =
            p->have_gpu && !fp32 ? decode_blocks_per_cu(desc->head_dim, f16, kvf, nw) : 0;
        p->grid_blocks = p->num_cus * (per_cu > 0 ? (nw == 1 ? std::max(per_cu, 8) : per_cu)
                                                  : (fp32 ? 2 : 8 / nw));
        // one chunk per resident work item (workgroup): a second, partial
        // round of chunks or chunks of a few blocks each measured slower
        p->auto_target_items = int64_t(p->num_cus) * (per_cu > 0 ? per_cu : std::max(1, 4 / nw));
    }
    (void)hipGetLastError();
    size_plan(p);
    if (fp32 && desc->kind == PKVS_DECODE) {
        // the fp32 path runs decode as one-token prefill items
        p->items_cap = int64_t(desc->batch_capacity) * desc->num_kv_heads;
        p->slots_cap = p->merges_cap = 0;
        p->int_ws_need = sizeof(int32_t) * size_t(kHeaderWords + p->items_cap * kPrefillItemWords);
        p->float_ws_need = 0;
    }
    p->grid_blocks = int32_t(std::max<int64_t>(1, std::min<int64_t>(p->grid_blocks, p->items_cap)));
    // A 16-bit decode plan gets everything a plan() call of its capacities
    // needs on the host here, once -- the planning buffers and the pinned
    // staging ring of the work-list copy -- so that planning and running a
    // decode batch allocate nothing (pkvs_decode_noalloc relies on it).
    if (desc->kind == PKVS_DECODE && !fp32 && make_buffers) {
        p->reqs_buf.reserve(size_t(desc->batch_capacity));
        p->req_slot.reserve(size_t(desc->batch_capacity));
        p->req_chunks.reserve(size_t(desc->batch_capacity));
        p->order_key.reserve(size_t(p->items_cap));
        p->pair_req.reserve(size_t(p->items_cap));
        p->pair_chunk.reserve(size_t(p->items_cap));
        p->merge_buf.reserve(size_t(p->merges_cap * kMergeWords));
        p->host_ws.reserve(p->int_ws_need / sizeof(int32_t));
        if (p->have_gpu) {
            const int rc = make_staging(p);
            if (rc) {
                destroy_plan(p);
                return rc;
            }
        }
    }
    *out = p;
    return PKVS_OK;
}

static void destroy_plan(Plan *p)
{
    if (!p) return;
    destroy_plan(p->ext);
    destroy_plan(p->pre);
    for (int i = 0; i < kStages; ++i) {
        if (p->stage_ev[i]) {
            if (p->stage_used[i]) (void)hipEventSynchronize(p->stage_ev[i]);
            (void)hipEventDestroy(p->stage_ev[i]);
        }
        if (p->stage[i]) (void)hipHostFree(p->stage[i]);
    }
    delete p;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// A cascade prefill is two prefill passes and one merge ([FIB]
// FlashInferAttnBackend.forward_extend, the branch for requests with a cached
// prefix).  The extend pass attends each request's new tokens to their own
// keys, read from a contiguous K/V (causal, with the window); the prefix pass
// attends them to the cached keys of the page table.  Every cached key comes
// before every new token, so there only the window's left edge hides keys
// ([FIB] FlashInferIndicesUpdaterPrefill._build_swa_prefix_custom_mask:
// visible iff k_abs >= q_abs - window).  merge_state combines the two (o, lse)
// pairs: the prefix pass runs first and leaves its (o, lse) in the float
// workspace, and the extend pass folds them into its own in its epilogue.
static int create_cascade(const pkvs_desc *desc, Plan **out)
{
    // One pass when a kernel that reads split key ranges (the default 64-key
    // kernel, or the register-staged 128- and 256-row ones) serves the
    // combined problem: each request's cached keys followed by its new tokens
    // form one causal sequence (cached key j at position j, new token i at
    // kv_len_b + i), and the window mask over it is exactly the pair of masks
    // the two passes apply; the kernel reads keys before a request's split
    // from the cache and the rest from the contiguous new-token K/V.
    if (desc->kv_format == PKVS_KV_SAME && desc->dtype != PKVS_FP32 &&
        desc->kv_capacity + desc->qo_capacity <= (int64_t(1) << 30)) {
        // (the cascade's own causality: causal, the window mask described
        // above; non-causal (no window), every key of the sequence)
        pkvs_desc f = *desc;
        f.kind = PKVS_PREFILL;
        f.kv_capacity = desc->kv_capacity + desc->qo_capacity;
        Plan *fp = nullptr;
        if (create_plan(&f, false, &fp) == PKVS_OK &&
            (fp->prefill_variant == kPrefillBig || fp->prefill_variant == kPrefillRows128 ||
             fp->prefill_variant == kPrefillRows256)) {
            Plan *p = new (std::nothrow) Plan();
            if (!p) {
                destroy_plan(fp);
                return fail(PKVS_ERR_INVALID_ARG, "out of host memory");
            }
            p->desc = *desc;
            p->fused = true;
            p->pre = fp;
            p->device = fp->device;
            p->have_gpu = fp->have_gpu;
            p->num_cus = fp->num_cus;
            p->grid_blocks = fp->grid_blocks;
            p->block_threads = fp->block_threads;
            p->query_tile = fp->query_tile;
            p->item_words = fp->item_words;
            p->prefill_variant = fp->prefill_variant;
            p->items_cap = fp->items_cap;
            p->int_ws_need = fp->int_ws_need;
            // (the partial slots of a key-split plan; 0 otherwise)
            p->float_ws_need = fp->float_ws_need;
            *out = p;
            return PKVS_OK;
        }
        destroy_plan(fp);
        clear_error();
    }
    pkvs_desc e = *desc, r = *desc;
    e.kind = r.kind = PKVS_PREFILL;
    e.page_size = kRaggedPage;          // row-index table entries
    e.kv_capacity = desc->qo_capacity;  // a request's extend keys are its queries
    e.kv_format = PKVS_KV_SAME;         // the new tokens' K/V come in the query dtype
    r.causal = 1;                       // the causal bound never hides a cached key
    Plan *p = new (std::nothrow) Plan();
    if (!p) return fail(PKVS_ERR_INVALID_ARG, "out of host memory");
    p->desc = *desc;
    int rc = create_plan(&e, true, &p->ext);
    // (the prefix pass writes the (o, lse) the extend pass folds: no key split)
    if (!rc) rc = create_plan(&r, false, &p->pre, true, false);
    if (rc) {
        destroy_plan(p);
        return rc;
    }
    const Plan *q = p->pre;
    p->pre->queries_after_kv = true;
    p->device = q->device;
    p->have_gpu = q->have_gpu;
    p->num_cus = q->num_cus;
    p->grid_blocks = q->grid_blocks;
    p->block_threads = q->block_threads;
    p->query_tile = q->query_tile;
    p->item_words = q->item_words;
    p->prefill_variant = q->prefill_variant;
    p->items_cap = p->ext->items_cap + q->items_cap;
    p->pre_int_off = align256(p->ext->int_ws_need);
    p->int_ws_need = p->pre_int_off + q->int_ws_need;
    const size_t esz = desc->dtype == PKVS_FP32 ? 4 : 2;
    const size_t rows = size_t(desc->qo_capacity) * size_t(desc->num_qo_heads);
    p->o2_off = 0;
    p->lse2_off = align256(rows * size_t(desc->head_dim) * esz);
    p->float_ws_need = p->lse2_off + rows * sizeof(float);
    *out = p;
    return PKVS_OK;
}

}  // namespace pkvs

using namespace pkvs;

extern "C" {

int pkvs_plan_create(pkvs_plan **out, const pkvs_desc *desc)
{
    clear_error();
    if (!out) return fail(PKVS_ERR_INVALID_ARG, "out is null");
    *out = nullptr;
    int rc = validate_desc(desc);
    if (rc) return rc;
    return desc->kind == PKVS_CASCADE ? create_cascade(desc, out) : create_plan(desc, false, out);
}

int pkvs_workspace_size(const pkvs_plan *p, size_t *float_ws_bytes, size_t *int_ws_bytes)
{
    clear_error();
    if (!p || !float_ws_bytes || !int_ws_bytes) return fail(PKVS_ERR_INVALID_ARG, "null argument");
    *float_ws_bytes = p->float_ws_need;
    *int_ws_bytes = p->int_ws_need;
    return PKVS_OK;
}

int pkvs_workspace_bytes(const pkvs_desc *desc, int32_t is_decode, int64_t max_kv_len,
                         size_t *float_ws_bytes, size_t *int_ws_bytes)
{
    clear_error();
    if (!desc || !float_ws_bytes || !int_ws_bytes)
        return fail(PKVS_ERR_INVALID_ARG, "null argument");
    if ((is_decode != 0) != (desc->kind == PKVS_DECODE))
        return fail(PKVS_ERR_INVALID_ARG, "is_decode %d disagrees with desc->kind %d",
                    is_decode, desc->kind);
    if (max_kv_len < 0) return fail(PKVS_ERR_INVALID_ARG, "max_kv_len %lld < 0",
                                    (long long)max_kv_len);
    pkvs_desc d = *desc;
    if (max_kv_len > 0) d.kv_capacity = max_kv_len;
    int rc = validate_desc(&d);
    if (rc) return rc;
    // (sizes only: no planning buffers or staging ring)
    pkvs_plan *p = nullptr;
    rc = d.kind == PKVS_CASCADE ? create_cascade(&d, &p) : create_plan(&d, false, &p, false);
    if (rc) return rc;
    *float_ws_bytes = p->float_ws_need;
    *int_ws_bytes = p->int_ws_need;
    destroy_plan(p);
    return PKVS_OK;
}

int pkvs_prefill_plan(pkvs_plan *p, const int32_t *qo_indptr_h, const int32_t *kv_indptr_h,
                      const int32_t *kv_last_page_len_h, int32_t batch_size, void *float_ws,
                      size_t float_ws_bytes, void *int_ws, size_t int_ws_bytes,
                      hipStream_t stream)
{
    clear_error();
    if (!p) return fail(PKVS_ERR_INVALID_ARG, "plan is null");
    if (p->desc.kind != PKVS_PREFILL) return fail(PKVS_ERR_INVALID_ARG, "not a prefill plan");
    p->planned_device = false;
    std::vector<Req> reqs;
    int rc = read_layout(p, qo_indptr_h, kv_indptr_h, kv_last_page_len_h, batch_size, reqs);
    if (rc) return rc;
    rc = build_prefill(p, reqs);
    if (rc) return rc;
    if (p->n_items > p->items_cap)
        return fail(PKVS_ERR_CAPACITY, "prefill work list of %lld items exceeds capacity %lld",
                    (long long)p->n_items, (long long)p->items_cap);
    p->batch = batch_size;
    return finish_plan(p, float_ws, float_ws_bytes, int_ws, int_ws_bytes, stream);
}

int pkvs_decode_plan(pkvs_plan *p, const int32_t *kv_indptr_h, const int32_t *kv_last_page_len_h,
                     int32_t batch_size, void *float_ws, size_t float_ws_bytes, void *int_ws,
                     size_t int_ws_bytes, hipStream_t stream)
{
    clear_error();
    if (!p) return fail(PKVS_ERR_INVALID_ARG, "plan is null");
    if (p->desc.kind != PKVS_DECODE) return fail(PKVS_ERR_INVALID_ARG, "not a decode plan");
    p->planned_device = false;
    std::vector<Req> &reqs = p->reqs_buf;
    int rc = read_layout(p, nullptr, kv_indptr_h, kv_last_page_len_h, batch_size, reqs);
    if (rc) return rc;
    if (p->desc.dtype == PKVS_FP32) {
        // one-token prefill items: query b at position kv_len-1
        std::vector<Req> as_prefill = reqs;
        for (size_t b = 0; b < reqs.size(); ++b) {
            as_prefill[b].qo_begin = int64_t(b);
            as_prefill[b].qo_len = 1;
        }
        // a keyless request still owns its query row: it becomes an item with
        // an empty key range, which writes o = 0 and lse = -inf
        rc = build_prefill(p, as_prefill);
        if (rc) return rc;
        p->split_size = 0;
    } else {
        rc = build_decode(p, reqs);
        if (rc) return rc;
    }
    if (p->n_items > p->items_cap)
        return fail(PKVS_ERR_CAPACITY, "decode work list of %lld items exceeds capacity %lld",
                    (long long)p->n_items, (long long)p->items_cap);
    p->batch = batch_size;
    return finish_plan(p, float_ws, float_ws_bytes, int_ws, int_ws_bytes, stream);
}

int pkvs_cascade_plan(pkvs_plan *p, const int32_t *qo_indptr_h, const int32_t *kv_indptr_h,
                      const int32_t *kv_last_page_len_h, int32_t batch_size, void *float_ws,
                      size_t float_ws_bytes, void *int_ws, size_t int_ws_bytes,
                      hipStream_t stream)
{
    clear_error();
    if (!p) return fail(PKVS_ERR_INVALID_ARG, "plan is null");
    if (p->desc.kind != PKVS_CASCADE) return fail(PKVS_ERR_INVALID_ARG, "not a cascade plan");
    p->planned_device = false;
    if (p->fused) {
        // the cached layout, read with the cascade's own rules (a request may
        // have more new tokens than cached keys), then each request as one
        // prefill request over its cached keys followed by its new tokens
        Plan lay;
        lay.desc = p->desc;
        lay.desc.kind = PKVS_PREFILL;
        lay.queries_after_kv = true;
        std::vector<Req> reqs;
        int rc = read_layout(&lay, qo_indptr_h, kv_indptr_h, kv_last_page_len_h, batch_size,
                             reqs);
        if (rc) return rc;
        int64_t cached = 0;
        for (Req &q : reqs) {
            cached += q.kv_len;
            q.split = q.kv_len;
            q.kv_len += q.qo_len;
        }
        Plan *f = p->pre;
        f->planned_device = false;
        rc = build_prefill(f, reqs);
        if (rc) return rc;
        if (f->n_items > f->items_cap)
            return fail(PKVS_ERR_CAPACITY, "cascade work list of %lld items exceeds capacity %lld",
                        (long long)f->n_items, (long long)f->items_cap);
        p->n_items = f->n_items;
        p->n_merges = f->n_merges;
        p->planned_keys = cached;
        p->batch = f->batch = batch_size;
        rc = finish_plan(f, float_ws, float_ws_bytes, int_ws, int_ws_bytes, stream);
        if (rc || !int_ws) return rc;
        p->int_ws = int_ws;
        p->float_ws = float_ws;
        p->planned_device = true;
        return PKVS_OK;
    }
    Plan *e = p->ext, *r = p->pre;
    e->planned_device = r->planned_device = false;
    std::vector<Req> pre_reqs;
    int rc = read_layout(r, qo_indptr_h, kv_indptr_h, kv_last_page_len_h, batch_size, pre_reqs);
    if (rc) return rc;
    // extend keys of request b: rows qo_begin .. qo_begin + qo_len - 1 of the
    // contiguous K/V, reached through table entries page_base ..
    std::vector<Req> ext_reqs(pre_reqs.size());
    int64_t entries = 0;
    for (size_t b = 0; b < pre_reqs.size(); ++b) {
        const Req &q = pre_reqs[b];
        ext_reqs[b] = Req{q.qo_begin, q.qo_len, q.qo_len, entries};
        entries += ceil_div(q.qo_len, kRaggedPage);
    }
    rc = build_prefill(e, ext_reqs);
    if (!rc) rc = build_prefill(r, pre_reqs);
    if (rc) return rc;
    if (e->n_items > e->items_cap || r->n_items > r->items_cap)
        return fail(PKVS_ERR_CAPACITY, "cascade work lists (%lld, %lld items) exceed capacity "
                    "(%lld, %lld)", (long long)e->n_items, (long long)r->n_items,
                    (long long)e->items_cap, (long long)r->items_cap);
    p->n_items = e->n_items + r->n_items;
    p->planned_keys = r->planned_keys;
    p->batch = e->batch = r->batch = batch_size;
    if (!int_ws) return PKVS_OK;  // dry plan
    if (int_ws_bytes < p->int_ws_need)
        return fail(PKVS_ERR_WORKSPACE, "int workspace %zu bytes < required %zu; increase the "
                    "workspace buffer size", int_ws_bytes, p->int_ws_need);
    if (!float_ws || float_ws_bytes < p->float_ws_need)
        return fail(PKVS_ERR_WORKSPACE, "float workspace %zu bytes < required %zu; increase "
                    "the workspace buffer size", float_ws ? float_ws_bytes : 0, p->float_ws_need);
    if (reinterpret_cast<uintptr_t>(float_ws) & 15)
        return fail(PKVS_ERR_INVALID_ARG, "the workspaces must be 16-byte aligned");
    rc = finish_plan(e, nullptr, 0, int_ws, p->pre_int_off, stream);
    if (!rc)
        rc = finish_plan(r, nullptr, 0, static_cast<char *>(int_ws) + p->pre_int_off,
                         int_ws_bytes - p->pre_int_off, stream);
    if (rc) return rc;
    p->int_ws = int_ws;
    p->float_ws = float_ws;
    p->planned_device = true;
    return PKVS_OK;
}

int pkvs_plan_get_info(const pkvs_plan *p, pkvs_plan_info *info)
{
    clear_error();
    if (!p || !info) return fail(PKVS_ERR_INVALID_ARG, "null argument");
    info->num_items = p->n_items;
    info->num_merges = p->n_merges;
    info->float_ws_bytes = int64_t(p->float_ws_need);
    info->int_ws_bytes = int64_t(p->int_ws_need);
    info->grid_blocks = p->grid_blocks;
    info->block_threads = p->block_threads;
    info->split_size = p->split_size;
    info->item_words = p->item_words;
    info->query_tile = p->query_tile;
    info->prefill_variant = p->desc.kind != PKVS_DECODE ? p->prefill_variant : 0;
    info->num_cus = p->num_cus;
    info->decode_waves = p->desc.kind == PKVS_DECODE ? p->decode_waves : 0;
    info->cascade_passes = p->desc.kind != PKVS_CASCADE ? 0 : p->fused ? 1 : 2;
    info->key_chunks = p->desc.kind == PKVS_DECODE ? 1
                       : p->desc.kind == PKVS_CASCADE && p->fused ? p->pre->key_chunks_max
                                                                  : p->key_chunks_max;
    return PKVS_OK;
}

int pkvs_plan_copy_items(const pkvs_plan *p, int32_t *dst, int64_t max_items, int64_t *n_items)
{
    clear_error();
    if (!p || !n_items) return fail(PKVS_ERR_INVALID_ARG, "null argument");
    *n_items = p->n_items;
    if (!dst) return PKVS_OK;
    // a cascade lists its extend pass's items, then its prefix pass's
    const Plan *parts[2] = {p, nullptr};
    if (p->desc.kind == PKVS_CASCADE) {
        parts[0] = p->ext;
        parts[1] = p->pre;
    }
    int64_t done = 0;
    for (const Plan *s : parts) {
        if (!s) continue;
        const int64_t n = std::min(max_items - done, s->n_items);
        if (n <= 0) break;
        std::memcpy(dst + done * s->item_words, s->host_ws.data() + s->lead_words + kHeaderWords,
                    sizeof(int32_t) * n * s->item_words);
        done += n;
    }
    return PKVS_OK;
}

void pkvs_plan_destroy(pkvs_plan *p) { destroy_plan(p); }

const char *pkvs_strerror(int code)
{
    switch (code) {
    case PKVS_OK: return "ok";
    case PKVS_ERR_INVALID_ARG: return "invalid argument";
    case PKVS_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKVS_ERR_WORKSPACE: return "workspace too small";
    case PKVS_ERR_CAPACITY: return "batch exceeds plan capacity";
    case PKVS_ERR_PLAN_MISMATCH: return "run arguments differ from the plan";
    case PKVS_ERR_HIP: return "HIP runtime error";
    case PKVS_ERR_NOT_PLANNED: return "no device plan";
    default: return "unknown status";
    }
}

const char *pkvs_last_error(void) { return g_last_error.c_str(); }

const char *pkvs_last_error_message(void) { return g_last_error.c_str(); }

}  // extern "C"
