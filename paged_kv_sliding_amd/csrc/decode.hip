// decode.hip -- single-token paged decode with grouped query heads, bf16,
// for gfx950.
//
// One wavefront owns one work item: (request, kv head, chunk of keys).  The
// G query heads that share the kv head are packed into the N dimension of
// 16x16x32 bf16 MFMAs, so each K/V byte is fetched once and serves all G
// heads (the reason sglang's should_use_tensor_core picks tensor cores for
// groups of 4 or more: the head group is fused with the token dimension).
//
// Per 32-key block:
//   S^T[16 keys x 16 heads] = K[16 keys x D] . Q^T[D x 16 heads]   (x2)
//       A operand: lane (row r = lane%16, group g = lane/16) holds 8 dims of
//       key r, read straight from the paged cache (dims 32s+8g.. at k-step s);
//       B operand: the same dims of query head r, kept in registers.
//   O^T[16 dims x 16 heads] += V^T[16 dims x 32 keys] . P^T[32 keys x 16 heads]
//       B operand: the probabilities exactly where the S^T accumulator left
//       them -- lane (head r, group g) holds keys 4g..4g+3 of both 16-key
//       halves, and those 8 keys are its 8 k-slots;
//       A operand: lane (r, g) loads dims 8r..8r+7 of those same 8 keys (eight
//       16-byte row loads) and transposes the 8x8 block in registers, which
//       gives it the A operand of 8 MFMAs at once (tile e holds dims 8r+e).
// So the kernel needs no LDS and no barrier, reads every K/V row with whole
// 16-byte loads, and applies the window as an exact per-key predicate.
//
// The window (AMD-Ecosystem/flashinfer PR 234, "Why each fix" 1): the query
// at kv_len-1 sees keys kv_len-1-W .. kv_len-1.  The planner only cuts the key
// range into chunks (sglang FlashInferIndicesUpdaterDecode.update_sliding_window
// trims it to the last W+1 keys); keys before the window start or past the
// chunk end are masked here, element by element.
//
// A chunk of a split request writes its fp32 partial (o normalised by its own
// sum, lse) to a slot of the float workspace; decode_merge combines them.
#include <type_traits>

#include "device_common.h"
#include "pkvs_internal.h"

namespace pkvs {

namespace {

// K and V rows are streamed once per work item and never re-read by it:
// non-temporal loads keep them from displacing other lines in the caches.
__device__ __forceinline__ bf16x8 load_stream(const void *p)
{
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}

__device__ __forceinline__ u32x2 load_stream8(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

__device__ __forceinline__ u32x4 load_stream16(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Loaded K/V of one 32-key block, as stored, widened where they are used.
// V: 8 elements per slot (16 bytes of a 16-bit cache, 8 of an 8-bit one).
// K: a 16-bit slot holds the 8 dims of one k-step; an 8-bit slot holds 16
// contiguous bytes, the dims of two k-steps (k-step 2t+h of lane group g
// takes dims 64t + 16g + 8h ..+7; the query operand uses the same map), so
// every K load moves 16 bytes per lane.
template <int D, int KVF>
struct DecodeBuf {
    static constexpr int KS = D / 32;            // QK k-steps (32 dims each)
    static constexpr int NV = D >= 128 ? D / 128 : 1;
    static constexpr int KN = KVF == 0 ? KS : KS / 2;  // K slots per key row
    using Raw = typename std::conditional<KVF == 0, bf16x8, u32x2>::type;
    using KRaw = typename std::conditional<KVF == 0, bf16x8, u32x4>::type;
    KRaw k0[KN], k1[KN];                         // keys blk+r, blk+16+r
    Raw v[NV][8];                                // 8 keys x 8 dims per 128-dim chunk
};

// first dim of k-step s for lane group g (see DecodeBuf)
template <int KVF>
__device__ __forceinline__ int kstep_dim(int s, int g)
{
    return KVF == 0 ? 32 * s + 8 * g : 64 * (s >> 1) + 16 * g + 8 * (s & 1);
}

// the K operand of k-step s from a key's slots
template <int D, bool F16, int KVF>
__device__ __forceinline__ bf16x8 k_operand(const typename DecodeBuf<D, KVF>::KRaw (&k)[DecodeBuf<D, KVF>::KN],
                                            int s)
{
    if constexpr (KVF == 0) {
        return k[s];
    } else {
        const u32x4 x = k[s >> 1];
        const u32x2 h = (s & 1) ? u32x2{x[2], x[3]} : u32x2{x[0], x[1]};
        return widen_fp8<KVF, F16>(h);
    }
}

template <bool F16, int KVF>
__device__ __forceinline__ bf16x8 widen_slot(const typename DecodeBuf<64, KVF>::Raw &x)
{
    if constexpr (KVF == 0) return x;
    else return widen_fp8<KVF, F16>(x);
}

// Page ids of a request, 64 pages at a time: lane L holds the id of page
// base + L (cur) and of page base + 64 + L (nxt, prefetched a window ahead).
// Windows start at a multiple of 32 keys and span 64 * page_size keys, so a
// 32-key block never straddles two windows.  Ids are fetched from the
// window with a cross-lane read, which keeps the dependent index loads off
// the critical path of the K/V stream.
struct PageWindow {
    int base, last_pg, page_base;
    int cur, nxt;
};

// Every load of the block loop is issued unconditionally (indexes clamped),
// so each block issues the same number of vector memory instructions and the
// compiler can wait for a block's own loads only, with the blocks behind it
// still in flight.
__device__ __forceinline__ int load_page_id(const DecodeArgs &a, const PageWindow &pw, int pg)
{
    return a.kv_indices[pw.page_base + min(pg, pw.last_pg)];
}

// The window moves (a wave-uniform decision) when a block's first key leaves
// it; the ids of the window after the current one are re-read on every block
// (the same ids until it moves).  The empty asm keeps the move a branch: as a
// select it would wait for the latest id load on every block.
__device__ __forceinline__ void window_advance(const DecodeArgs &a, PageWindow &pw, int key,
                                               int lane)
{
    if ((key >> a.log2_page) - pw.base >= 64) {
        pw.base += 64;
        pw.cur = pw.nxt;
        asm volatile("" : "+v"(pw.cur));
    }
    pw.nxt = load_page_id(a, pw, pw.base + 64 + lane);
}

__device__ __forceinline__ int64_t clamp_page(const DecodeArgs &a, int64_t pg)
{
    pg = pg < 0 ? 0 : pg;
    return pg >= a.num_pages ? a.num_pages - 1 : pg;
}

// page of key `tok` (any lane's own key): a cross-lane read of the window
__device__ __forceinline__ int64_t window_page(const DecodeArgs &a, const PageWindow &pw, int tok)
{
    return clamp_page(a, __shfl(pw.cur, (tok >> a.log2_page) - pw.base));
}

// page of key `tok`, the same for every lane: a scalar read of the window
__device__ __forceinline__ int64_t window_page_uniform(const DecodeArgs &a, const PageWindow &pw,
                                                       int tok)
{
    const int idx = __builtin_amdgcn_readfirstlane((tok >> a.log2_page) - pw.base);
    return clamp_page(a, __builtin_amdgcn_readlane(pw.cur, idx & 63));
}

// Byte offsets of a lane's loads within a 16-key half of a block, from the
// half's first key row (this kv head), the same for every block: K row r
// (bytes 16g.. of each 64-byte k-step group), V rows 4g+i (dims dv..).
struct LaneOffsets {
    uint32_t k;
    uint32_t v[4];
};

template <int D, int KVF>
__device__ __forceinline__ LaneOffsets lane_offsets(const DecodeArgs &a, int lane)
{
    constexpr int esz = KVF == 0 ? 2 : 1;
    const int r = lane & 15, g = lane >> 4;
    const uint32_t slot_bytes = uint32_t(a.num_kv_heads) * D * esz;
    LaneOffsets lo;
    lo.k = uint32_t(r) * slot_bytes + 16u * uint32_t(g);
    const uint32_t dv = uint32_t(min(8 * r, D - 8)) * esz;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo.v[i] = uint32_t(4 * g + i) * slot_bytes + dv;
    return lo;
}

template <int D, int KVF>
__device__ __forceinline__ void decode_load(DecodeBuf<D, KVF> &buf, const DecodeArgs &a,
                                            PageWindow &pw, int blk, int t1, int hk, int lane,
                                            const LaneOffsets &lo)
{
    using Buf = DecodeBuf<D, KVF>;
    constexpr int KS = Buf::KS, NV = Buf::NV;
    using Elem = typename std::conditional<KVF == 0, uint16_t, uint8_t>::type;
    constexpr int esz = int(sizeof(Elem));
    const int r = lane & 15, g = lane >> 4;
    const int P = a.page_size;
    const Elem *K = static_cast<const Elem *>(a.k);
    const Elem *V = static_cast<const Elem *>(a.v);
    const int last = t1 - 1;
    // blocks past the end read the request's last key; the window never moves
    // past its page
    window_advance(a, pw, min(blk, last), lane);
    auto load = [](const void *p) __attribute__((always_inline)) {
        if constexpr (KVF == 0) return load_stream(p);
        else return load_stream8(p);
    };

    if (P >= 16 && blk + kDecodeBlock <= t1) {
        // A whole block with 16-key pages: each half is 16 consecutive rows of
        // one page, so every load is a wave-uniform half base (page id read
        // from the window, scalar arithmetic) plus the lane's fixed offset.
        const int64_t slot_bytes = int64_t(a.num_kv_heads) * D * esz;
        const int64_t page_bytes = slot_bytes * P;
        const int64_t head_bytes = int64_t(hk) * D * esz;
        const int64_t ha = window_page_uniform(a, pw, blk) * page_bytes + head_bytes +
                           int64_t(blk & (P - 1)) * slot_bytes;
        const int64_t hb = window_page_uniform(a, pw, blk + 16) * page_bytes + head_bytes +
                           int64_t((blk + 16) & (P - 1)) * slot_bytes;
        const char *const Ka = reinterpret_cast<const char *>(K) + ha;
        const char *const Kb = reinterpret_cast<const char *>(K) + hb;
        const char *const Va = reinterpret_cast<const char *>(V) + ha;
        const char *const Vb = reinterpret_cast<const char *>(V) + hb;
        if constexpr (KVF == 0) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                buf.k0[s] = load_stream(Ka + lo.k + 64 * s);
                buf.k1[s] = load_stream(Kb + lo.k + 64 * s);
            }
        } else {
#pragma unroll
            for (int t = 0; t < Buf::KN; ++t) {
                buf.k0[t] = load_stream16(Ka + lo.k + 64 * t);
                buf.k1[t] = load_stream16(Kb + lo.k + 64 * t);
            }
        }
#pragma unroll
        for (int u = 0; u < NV; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const typename Buf::Raw xa = load(Va + lo.v[i] + 128 * esz * u);
                const typename Buf::Raw xb = load(Vb + lo.v[i] + 128 * esz * u);
                const typename Buf::Raw z = {};
                buf.v[u][i] = (8 * r + 128 * u < D) ? xa : z;
                buf.v[u][4 + i] = (8 * r + 128 * u < D) ? xb : z;
            }
        return;
    }

    // key rows of the A operand of S^T: keys blk+r and blk+16+r;
    // value rows: keys blk+4g+i and blk+16+4g+i (i = 0..3), dims 8r..8r+7
    const int tk0 = min(blk + r, last), tk1 = min(blk + 16 + r, last);
    const int64_t head = int64_t(hk) * D;
    const int64_t slot_stride = int64_t(a.num_kv_heads) * D;
    int64_t rk0, rk1, rv[8];
    if (P >= 16) {
        // a block starts at a multiple of 32 keys, so each 16-key half lies in
        // one page: two wave-uniform page ids per block, scalar address bases
        const int64_t page_stride = slot_stride * P;
        const int64_t ba = window_page_uniform(a, pw, min(blk, last)) * page_stride + head;
        const int64_t bb = window_page_uniform(a, pw, min(blk + 16, last)) * page_stride + head;
        rk0 = ba + (tk0 & (P - 1)) * slot_stride;
        rk1 = bb + (tk1 & (P - 1)) * slot_stride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sa = min(blk + 4 * g + i, last), sb = min(blk + 16 + 4 * g + i, last);
            rv[i] = ba + (sa & (P - 1)) * slot_stride;
            rv[4 + i] = bb + (sb & (P - 1)) * slot_stride;
        }
    } else {
        rk0 = nhd_offset(window_page(a, pw, tk0), tk0 & (P - 1), P, hk, a.num_kv_heads, D);
        rk1 = nhd_offset(window_page(a, pw, tk1), tk1 & (P - 1), P, hk, a.num_kv_heads, D);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = min(blk + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4), last);
            rv[j] = nhd_offset(window_page(a, pw, t), t & (P - 1), P, hk, a.num_kv_heads, D);
        }
    }
    if constexpr (KVF == 0) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            buf.k0[s] = load_stream(K + rk0 + 32 * s + 8 * g);
            buf.k1[s] = load_stream(K + rk1 + 32 * s + 8 * g);
        }
    } else {
#pragma unroll
        for (int t = 0; t < Buf::KN; ++t) {
            buf.k0[t] = load_stream16(K + rk0 + 64 * t + 16 * g);
            buf.k1[t] = load_stream16(K + rk1 + 64 * t + 16 * g);
        }
    }
    // (D = 64: lanes r >= 8 read a valid slice of the row and drop it)
    const int dv = min(8 * r, D - 8);
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const typename Buf::Raw x = load(V + rv[j] + 128 * u + dv);
            const typename Buf::Raw z = {};
            buf.v[u][j] = (8 * r + 128 * u < D) ? x : z;
        }
}

template <int D>
struct DecodeState {
    static constexpr int NV = DecodeBuf<D, 0>::NV;
    float m, l;
    f32x4 o[NV][8];
};

template <int D, bool F16, int KVF>
__device__ __forceinline__ void decode_compute(const DecodeBuf<D, KVF> &buf, DecodeState<D> &st,
                                               const bf16x8 (&qf)[D / 32], int blk, int lo,
                                               int t1, float scale_log2, float cap_a, int lane)
{
    constexpr int KS = DecodeBuf<D, KVF>::KS, NV = DecodeBuf<D, KVF>::NV;
    const int g = lane >> 4;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        s0 = mfma16x16x32<F16>(k_operand<D, F16, KVF>(buf.k0, s), qf[s], s0);
        s1 = mfma16x16x32<F16>(k_operand<D, F16, KVF>(buf.k1, s), qf[s], s1);
    }
    // lane holds keys blk+4g+i (s0[i]) and blk+16+4g+i (s1[i]) of head lane%16
    float x[8];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ta = blk + 4 * g + i, tb = blk + 16 + 4 * g + i;
        float ra = s0[i], rb = s1[i];
        if (cap_a != 0.f) {
            ra = soft_cap_unit(ra, cap_a);
            rb = soft_cap_unit(rb, cap_a);
        }
        x[i] = (ta >= lo && ta < t1) ? ra * scale_log2 : kNegInf;
        x[4 + i] = (tb >= lo && tb < t1) ? rb * scale_log2 : kNegInf;
        mx = fmaxf(mx, fmaxf(x[i], x[4 + i]));
    }
    // across the four lane groups: row swaps (VALU), no LDS round trip
    {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float m_new = fmaxf(st.m, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(st.m - m_use);
    float p[8], rs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        p[j] = fast_exp2(x[j] - m_use);
        rs += p[j];
    }
    st.l = st.l * alpha + rs;
    st.m = m_new;
    f32x8 pv = {p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
    const bf16x8 pb = to16x8<F16>(pv);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        bf16x8 vrow[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) vrow[j] = widen_slot<F16, KVF>(buf.v[u][j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x8 va;
#pragma unroll
            for (int j = 0; j < 8; ++j) va[j] = vrow[j][e];
            st.o[u][e] = mfma16x16x32<F16>(va, pb, st.o[u][e] * alpha);
        }
    }
}

// Register buffers in the pipeline.  16-bit K/V: D = 64 holds three 32-key
// buffers (two in flight while the third is consumed); D >= 128 holds two,
// one in flight while the other is consumed.  At D = 128 both fit one wave
// per SIMD, and the third buffer measured slower: it costs register moves in
// the loop and a longer pipeline fill at every item's start.  8-bit K/V moves
// half the bytes per key, so it holds one buffer more at each D.
template <int D, int KVF>
constexpr int decode_stages() { return KVF == 0 ? (D >= 128 ? 2 : 3) : (D >= 256 ? 3 : 4); }

// NS register buffers of 32 keys each: NS-1 blocks are in flight while one is
// being computed.
// NW waves share a work item: wave w streams the w-th of NW contiguous runs of
// the chunk's key blocks with its own running maximum, sum and O, and the
// waves combine them through LDS (the LSE-weighted sum of merge_state).  A
// batch of a few (request, kv head) pairs then needs 1/NW of the chunks, and
// of the partials and merge work, that it needs with one wave per item.
template <int D, int NW>
struct DecodeMergeLds {
    static constexpr int NV = DecodeBuf<D, 0>::NV;
    float m[NW][16], l[NW][16];
    float o[NW > 1 ? NW - 1 : 1][NW > 1 ? NV * 32 : 1][64];  // waves 1.., element, lane
    int32_t next_item;
};

template <int D, int NS, bool F16, int KVF, int NW>
__global__ __launch_bounds__(kDecodeThreads * NW) void decode_kernel(DecodeArgs a)
{
    constexpr int KS = D / 32, NV = DecodeBuf<D, KVF>::NV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : 0;
    const int r = lane & 15, g = lane >> 4;
    const int G = 1 << a.log2_group;
    const int n_items = a.ws[kHdrNumItems];
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    __shared__ DecodeMergeLds<D, NW> sh;

    // Items are handed out at run time: each workgroup starts with item
    // blockIdx.x and then takes the next untaken one from a counter in the
    // workspace header, so workgroups that stream faster take more items and
    // the launch ends when the slowest finishes its last item, not its fourth.
    // (One wave: claimed at the item's end; several: claimed by thread 0 at the
    // item's start and passed on through LDS at its end.)
    // With a workgroup for every item there is nothing to hand out: each takes
    // item blockIdx.x only and the counters are not touched (they stay 0).
    int32_t *const ctr = a.ws;
    const bool claiming = int(gridDim.x) < n_items;
    // Every processed item is followed (one wave) or preceded (several) by
    // exactly one claim, so a launch makes n_items claims, returning 0 ..
    // n_items-1: the workgroup that draws n_items-1 makes the launch's last
    // claim and puts the counter back to 0 for the next launch.
    auto next_item = [&]() __attribute__((always_inline)) {
        if (!claiming) return n_items;
        int v = 0;
        if (lane == 0) {
            v = atomicAdd(ctr + kHdrNextItem, 1);
            if (v == n_items - 1) ctr[kHdrNextItem] = 0;
        }
        return int(gridDim.x) + __builtin_amdgcn_readfirstlane(v);
    };
    // Workgroups past the item count have nothing to claim: they leave without
    // touching the counter.
    if (int(blockIdx.x) >= n_items) return;
    for (int it = blockIdx.x; it < n_items;) {
        int claimed = 0;
        if (NW > 1 && claiming && tid == 0) {
            claimed = atomicAdd(ctr + kHdrNextItem, 1);
            if (claimed == n_items - 1) ctr[kHdrNextItem] = 0;
        }
        const int32_t *w = a.ws + kHeaderWords + int64_t(it) * kDecodeItemWords;
        const int b = w[kDiRequest], hk = w[kDiKvHead];
        const int t0 = w[kDiTokBegin], t1 = w[kDiTokEnd], lo = w[kDiVisLo];
        const int page_base = w[kDiPageBase], slot = w[kDiSlot];
        // this wave's run of the chunk's key blocks: [s0, s1)
        const int nblk = t0 < t1 ? (t1 - t0 + kDecodeBlock - 1) / kDecodeBlock : 0;
        const int s0 = t0 + kDecodeBlock * (nblk * wave / NW);
        const int s1 = min(t1, t0 + kDecodeBlock * (nblk * (wave + 1) / NW));

        // Q^T operand: head r of the group, the dims of k-step s for lane
        // group g (kstep_dim; zero for padding heads)
        bf16x8 qf[KS];
        const int64_t qrow = (int64_t(b) * a.num_qo_heads + hk * G + r) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qf[s] = r < G ? load_bf16x8(Q + qrow + kstep_dim<KVF>(s, g)) : zero_bf16x8();

        DecodeState<D> st;
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int u = 0; u < NV; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) st.o[u][e] = f32x4{0.f, 0.f, 0.f, 0.f};

        if (s0 < s1) {
            PageWindow pw;
            pw.page_base = page_base;
            pw.base = __builtin_amdgcn_readfirstlane(s0 >> a.log2_page);
            pw.last_pg = (s1 - 1) >> a.log2_page;
            pw.cur = load_page_id(a, pw, pw.base + lane);
            pw.nxt = load_page_id(a, pw, pw.base + 64 + lane);
            DecodeBuf<D, KVF> buf[NS];
            const LaneOffsets loff = lane_offsets<D, KVF>(a, lane);
            // blocks past the end load the request's last key (clamped) and
            // are never computed
#pragma unroll
            for (int s = 0; s + 1 < NS; ++s)
                decode_load<D, KVF>(buf[s], a, pw, s0 + kDecodeBlock * s, s1, hk, lane, loff);
            int blk = s0;
            bool done = false;
            while (!done) {
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    decode_load<D, KVF>(buf[(s + NS - 1) % NS], a, pw, blk + kDecodeBlock * (NS - 1),
                                   s1, hk, lane, loff);
                    decode_compute<D, F16, KVF>(buf[s], st, qf, blk, lo, s1, a.scale_log2, a.cap_a, lane);
                    blk += kDecodeBlock;
                    if (blk >= s1) {
                        done = true;
                        break;
                    }
                }
            }
        }

        // the four lane groups hold disjoint keys of the same head: sum them
        float l = st.l, m = st.m;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if constexpr (NW > 1) {
            // every wave rescales its sum and O to the largest maximum; waves
            // 1.. leave O in LDS (element-major, lane-contiguous) for wave 0
            if (g == 0) {
                sh.m[wave][r] = m;
                sh.l[wave][r] = l;
            }
            __syncthreads();
            float mx = kNegInf;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) mx = fmaxf(mx, sh.m[w2][r]);
            const float mu = mx == kNegInf ? 0.f : mx;
            float lt = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) lt += sh.l[w2][r] * fast_exp2(sh.m[w2][r] - mu);
            const float f = fast_exp2(m - mu);
            if (wave > 0) {
#pragma unroll
                for (int u = 0; u < NV; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            sh.o[wave - 1][(u * 8 + e) * 4 + i][lane] = st.o[u][e][i] * f;
            }
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int u = 0; u < NV; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float acc = st.o[u][e][i] * f;
#pragma unroll
                            for (int w2 = 1; w2 < NW; ++w2) acc += sh.o[w2 - 1][(u * 8 + e) * 4 + i][lane];
                            st.o[u][e][i] = acc;
                        }
            }
            m = mx;
            l = lt;
        }
        const float inv = l > 0.f ? a.v_scale / l : 0.f;
        const float lse = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
        if (wave == 0 && r < G) {
            // O^T accumulator: lane (head r, group g) holds dims 128u+32g+8i+e
            const int h = hk * G + r;
            if (slot < 0) {
                uint16_t *O = static_cast<uint16_t *>(a.o);
                const int64_t orow = (int64_t(b) * a.num_qo_heads + h) * D;
#pragma unroll
                for (int u = 0; u < NV; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int d0 = 128 * u + 32 * g + 8 * i;
                        if (d0 < D) {
                            f32x8 ov;
#pragma unroll
                            for (int e = 0; e < 8; ++e) ov[e] = st.o[u][e][i] * inv;
                            *reinterpret_cast<bf16x8 *>(O + orow + d0) = to16x8<F16>(ov);
                        }
                    }
                if (a.lse && g == 0) a.lse[int64_t(b) * a.num_qo_heads + h] = lse;
            } else {
                float *PO = a.part_o + (int64_t(slot) * G + r) * D;
#pragma unroll
                for (int u = 0; u < NV; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int d0 = 128 * u + 32 * g + 8 * i;
                        if (d0 < D) {
                            f32x4 lo4, hi4;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                lo4[e] = st.o[u][e][i] * inv;
                                hi4[e] = st.o[u][e + 4][i] * inv;
                            }
                            *reinterpret_cast<f32x4 *>(PO + d0) = lo4;
                            *reinterpret_cast<f32x4 *>(PO + d0 + 4) = hi4;
                        }
                    }
                if (g == 0) a.part_lse[int64_t(slot) * G + r] = lse;
            }
        }
        if constexpr (NW > 1) {
            // also orders this item's LDS reads before the next item's writes
            if (tid == 0) sh.next_item = claiming ? int(gridDim.x) + claimed : n_items;
            __syncthreads();
            it = sh.next_item;
        } else {
            it = next_item();
        }
    }
}

// Combine the chunk partials of every split (request, kv head): one unit per
// (merge entry, query head of the group), the LSE-weighted sum of
// pkvs_merge_state folded over all chunks at once.  P16: the partial o is in
// the query dtype (part_o16; a key-split prefill's merge entries are (query
// token, kv head) pairs), else fp32.  A wave merges kMergeUnitsPerWave units
// at once, 64 / kMergeUnitsPerWave lanes each; lane i of a unit holds
// elements E i .. E i + E - 1 of the row, so each partial row is one
// contiguous load per lane, and the units' reads overlap.
template <int D, bool F16, bool P16>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a)
{
    constexpr int L = 64 / kMergeUnitsPerWave;  // lanes per unit
    constexpr int E = D / L;                    // elements per lane
    using P16v = uint16_t __attribute__((ext_vector_type(E)));
    using P32v = float __attribute__((ext_vector_type(E)));
    const int li = threadIdx.x % L, grp = threadIdx.x / L;
    const int G = 1 << a.log2_group;
    const int n_merges = a.ws[kHdrNumMerges];
    const int32_t *merges = a.ws + a.ws[kHdrMergeOffset];
    const int units = n_merges << a.log2_group;
    for (int u0 = blockIdx.x * kMergeUnitsPerWave; u0 < units;
         u0 += gridDim.x * kMergeUnitsPerWave) {
        const int u = u0 + grp;
        if (u >= units) continue;
        const int32_t *me = merges + (u >> a.log2_group) * kMergeWords;
        const int h = u & (G - 1);
        const int b = me[kMeRequest], hk = me[kMeKvHead], first = me[kMeFirstSlot],
                  n = me[kMeNumSlots];
        float M = kNegInf;
        for (int k = 0; k < n; ++k) M = fmaxf(M, a.part_lse[int64_t(first + k) * G + h]);
        float acc[E] = {};
        float sum = 0.f;
        if (M != kNegInf) {
            for (int k = 0; k < n; ++k) {
                const int64_t sl = int64_t(first + k) * G + h;
                const float wk = fast_exp2((a.part_lse[sl] - M) * 1.44269504088896340736f);
                sum += wk;
                if constexpr (P16) {
                    const P16v v = *reinterpret_cast<const P16v *>(a.part_o16 + sl * D + E * li);
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] += wk * from16<F16>(v[e]);
                } else {
                    const P32v v = *reinterpret_cast<const P32v *>(a.part_o + sl * D + E * li);
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] += wk * v[e];
                }
            }
        }
        const float inv = sum > 0.f ? 1.f / sum : 0.f;
        const int64_t orow = (int64_t(b) * a.num_qo_heads + hk * G + h) * D;
        P16v out;
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = to16<F16>(acc[e] * inv);
        *reinterpret_cast<P16v *>(static_cast<uint16_t *>(a.o) + orow + E * li) = out;
        if (a.lse && li == 0)
            a.lse[int64_t(b) * a.num_qo_heads + hk * G + h] =
                sum > 0.f ? M + fast_log2(sum) * kLn2 : kNegInf;
    }
}

}  // namespace

template <bool F16, int KVF, int NW>
static hipError_t launch_decode_w(const DecodeArgs &a, int head_dim, int grid, hipStream_t s)
{
    switch (head_dim) {
    case 64:
        decode_kernel<64, decode_stages<64, KVF>(), F16, KVF, NW><<<grid, kDecodeThreads * NW, 0, s>>>(a);
        break;
    case 128:
        decode_kernel<128, decode_stages<128, KVF>(), F16, KVF, NW><<<grid, kDecodeThreads * NW, 0, s>>>(a);
        break;
    case 256:
        decode_kernel<256, decode_stages<256, KVF>(), F16, KVF, NW><<<grid, kDecodeThreads * NW, 0, s>>>(a);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool F16, int KVF>
static hipError_t launch_decode_t(const DecodeArgs &a, int head_dim, int waves, int grid,
                                  hipStream_t s)
{
    switch (waves) {
    case 1: return launch_decode_w<F16, KVF, 1>(a, head_dim, grid, s);
    case 4: return launch_decode_w<F16, KVF, 4>(a, head_dim, grid, s);
    default: return hipErrorInvalidValue;
    }
}

template <bool F16>
static hipError_t launch_decode_f(const DecodeArgs &a, int head_dim, int kv_format, int waves,
                                  int grid, hipStream_t s)
{
    switch (kv_format) {
    case 0: return launch_decode_t<F16, 0>(a, head_dim, waves, grid, s);
    case PKVS_KV_FP8_E4M3: return launch_decode_t<F16, 1>(a, head_dim, waves, grid, s);
    case PKVS_KV_FP8_E5M2: return launch_decode_t<F16, 2>(a, head_dim, waves, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_16bit(const DecodeArgs &a, int head_dim, bool f16, int kv_format,
                               int waves, int grid, hipStream_t s)
{
    return f16 ? launch_decode_f<true>(a, head_dim, kv_format, waves, grid, s)
               : launch_decode_f<false>(a, head_dim, kv_format, waves, grid, s);
}

template <bool F16, bool P16>
static hipError_t launch_merge_t(const DecodeArgs &a, int head_dim, int grid, hipStream_t s)
{
    switch (head_dim) {
    case 64: decode_merge_kernel<64, F16, P16><<<grid, kMergeThreads, 0, s>>>(a); break;
    case 128: decode_merge_kernel<128, F16, P16><<<grid, kMergeThreads, 0, s>>>(a); break;
    case 256: decode_merge_kernel<256, F16, P16><<<grid, kMergeThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs &a, int head_dim, bool f16, bool p16, int grid,
                               hipStream_t s)
{
    if (p16)
        return f16 ? launch_merge_t<true, true>(a, head_dim, grid, s)
                   : launch_merge_t<false, true>(a, head_dim, grid, s);
    return f16 ? launch_merge_t<true, false>(a, head_dim, grid, s)
               : launch_merge_t<false, false>(a, head_dim, grid, s);
}

template <bool F16, int KVF, int NW>
static int decode_blocks_per_cu_w(int head_dim)
{
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (head_dim) {
    case 64:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, decode_kernel<64, decode_stages<64, KVF>(), F16, KVF, NW>, kDecodeThreads * NW, 0);
        break;
    case 128:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, decode_kernel<128, decode_stages<128, KVF>(), F16, KVF, NW>, kDecodeThreads * NW, 0);
        break;
    case 256:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, decode_kernel<256, decode_stages<256, KVF>(), F16, KVF, NW>, kDecodeThreads * NW, 0);
        break;
    }
    return e == hipSuccess ? n : 0;
}

template <bool F16, int KVF>
static int decode_blocks_per_cu_t(int head_dim, int waves)
{
    switch (waves) {
    case 1: return decode_blocks_per_cu_w<F16, KVF, 1>(head_dim);
    case 4: return decode_blocks_per_cu_w<F16, KVF, 4>(head_dim);
    default: return 0;
    }
}

template <bool F16>
static int decode_blocks_per_cu_f(int head_dim, int kv_format, int waves)
{
    switch (kv_format) {
    case 0: return decode_blocks_per_cu_t<F16, 0>(head_dim, waves);
    case PKVS_KV_FP8_E4M3: return decode_blocks_per_cu_t<F16, 1>(head_dim, waves);
    case PKVS_KV_FP8_E5M2: return decode_blocks_per_cu_t<F16, 2>(head_dim, waves);
    default: return 0;
    }
}

int decode_blocks_per_cu(int head_dim, bool f16, int kv_format, int waves)
{
    return f16 ? decode_blocks_per_cu_f<true>(head_dim, kv_format, waves)
               : decode_blocks_per_cu_f<false>(head_dim, kv_format, waves);
}

}  // namespace pkvs
