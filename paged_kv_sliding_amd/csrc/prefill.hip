// prefill.hip -- causal paged prefill (extend with a cached prefix) with the
// exact sliding-window mask, for gfx950.
//
// bf16 path: one workgroup of NW = 4 or 8 waves owns one work item =
// (request, kv head, tile of 32*NW/G query tokens).  The G query heads of the
// kv head are packed with the tokens into 32*NW rows (row = token * G + head),
// so a K/V tile staged in LDS serves all of them.  Each wave owns 32 rows and
// runs
//     S^T[32 keys x 32 rows] = K[32 keys x D] . Q^T[D x 32 rows]
//     O^T[32 dims x 32 rows] += V^T[32 dims x 32 keys] . P^T[32 keys x 32 rows]
// on v_mfma_f32_32x32x16_bf16.  With S^T (keys in M) every lane holds 16 keys
// of one row, so the row maximum and sum are lane-local plus one exchange
// with the lane 32 away, and the probabilities are already laid out as the B
// operand of the PV product.  K and V sit in LDS row-major; the V^T operand
// comes from gfx950's transposing LDS read.
//
// Four LDS tile sets are in flight (one barrier per tile): while tile j's
// softmax runs, the MFMAs of tile j+1's S^T are already issued, tile j+2 is
// being written to LDS and tile j+3 read from HBM into registers; with 8 waves
// the second half of the waves multiplies P.V one tile late (ping-pong), which
// keeps V of tile j-1 live in the fourth set.
// The running row maximum is only moved (and O rescaled) when it grows by more
// than 2^8, which most tiles never do.
//
// The key loop starts at the tile holding the window start of the item's
// first query (the per-tile KV-start skip of the planner) and stops at the
// tile holding its last query.  Tiles that straddle the window edge, the
// causal diagonal or the end of the keys get the per-element mask
//     key <= p  and  key >= p - window_left  and  key < kv_len
// (sglang PR "Pass window_left at plan time for the SWA paged prefill
// wrapper", section "What": the tile skip alone leaks keys); interior tiles
// are fully visible and skip the compare.
//
// Key split (prefill_kernel and prefill_big_kernel, batches of few query
// tiles): an item may be one chunk of a tile's key range, ending at a key
// tile boundary (kPiKvEnd); it then writes
// each row's partial (o normalised over its keys, in the query dtype; lse in
// fp32) to the float workspace for the per-token merge instead of o / lse.
//
// fp32 path (attention_fp32_kernel): a plain wave-per-row loop in fp32 for
// fp32 inputs, used for small correctness-critical problems; it serves both
// prefill items and decode (as one-query items).
#include <type_traits>

#include "device_common.h"
#include "pkvs_internal.h"

namespace pkvs {

namespace {

constexpr int KT = kPrefillKvTile;
constexpr int KPAD = 8;                // K rows: D+8 bf16, a stride of 4 dwords mod 64 banks
constexpr int VPAD = 32;               // V rows: D+32 bf16, a stride of 16 dwords mod 64 banks
constexpr int NBUF = 4;                // LDS tile sets in flight
constexpr float kRescaleLog2 = 8.0f;   // rescale O only when a row max grows by > 2^8

// Folding this pass's (o, lse) of a row into a second partial over other keys
// of the same query (sglang flashinfer_backend.py, _safe_merge_state):
// s = ln(e^s_self + e^s_other), o = e^(s_self - s) o_self + e^(s_other - s) o_other;
// two empty partials stay empty (o = 0, s = -inf).
struct Fold {
    float self, other, lse;
};

__device__ __forceinline__ Fold fold_weights(float s_self, float s_other)
{
    constexpr float kLog2e = 1.44269504088896340736f;
    const float M = fmaxf(s_self, s_other);
    if (M == kNegInf) return Fold{0.f, 0.f, kNegInf};
    const float ea = fast_exp2((s_self - M) * kLog2e), eb = fast_exp2((s_other - M) * kLog2e);
    const float sum = ea + eb;
    return Fold{ea / sum, eb / sum, M + fast_log2(sum) * kLn2};
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One key tile in LDS, K and V both row-major.  The A operand of S^T = K.Q^T
// is a plain 16-byte read of a key row.  The A operand of O^T = V^T.P^T needs
// 8 keys of one dim per lane; gfx950's transposing LDS read provides it: in
// each 16-lane group, the lane 4e+q that points at V[k0+e][d0+4q] makes lane
// i receive V[k0..k0+3][d0 + i mod 16].
template <int D>
struct PrefillBuf {
    uint16_t k[KT][D + KPAD];
    uint16_t v[KT][D + VPAD];
};

// Per-thread staging of one key tile: the NW*64 threads copy the tile's K and
// V rows in chunks of 8 elements (chunk c: key c / (D/8), dims 8*(c % (D/8)));
// 16 bytes from a 16-bit cache, 8 bytes from an 8-bit one (KVF != 0), widened
// to 16 bits on the way into LDS.  The page ids of a tile are read one tile
// before its K/V loads and kept raw: the address arithmetic that needs them
// runs only when the loads are issued, so no wait on the page-table read sits
// behind freshly issued K/V loads.
template <int D, int NW, int KVF>
struct Stage {
    static constexpr int T = NW * 64;
    static constexpr int NCH = KT * D / 8;          // chunks per tile and tensor
    static constexpr int KCH = (NCH + T - 1) / T;   // per thread
    using Raw = typename std::conditional<KVF == 0, u32x4, u32x2>::type;
    Raw k[KCH], v[KCH];
    int32_t page[KCH];  // page id of the chunk's key (next tile to load)
};

struct RowAddr {
    const int32_t *kv_indices;
    int64_t num_pages, page_stride, slot_stride, head_off;
    int page_base, log2_page, page_mask, kv_len;
    // one-pass cascade: keys from `split` on are new-token rows of the
    // contiguous K/V (key k on row k + ext_row0); INT32_MAX: none
    int split = INT32_MAX, ext_row0 = 0;

    __device__ __forceinline__ int clamp_key(int key) const { return min(key, kv_len - 1); }
    // (keys past the split have no page: their entry is never read)
    __device__ __forceinline__ int32_t page_id(int key) const
    {
        const int k = min(clamp_key(key), split - 1);
        return k < 0 ? 0 : kv_indices[page_base + (k >> log2_page)];
    }
    // element offset of `key` (clamped into the request) on page `pg`; the
    // planner keeps page_stride below 2^31, so one 32x32->64 multiply does
    __device__ __forceinline__ int64_t offset(int32_t pg, int key) const
    {
        const uint32_t p = uint32_t(min(max(pg, 0), int32_t(num_pages - 1)));
        return int64_t(uint64_t(p) * uint32_t(page_stride)) +
               int32_t((clamp_key(key) & page_mask) * int32_t(slot_stride) + int32_t(head_off));
    }
};

template <int D, int NW>
__device__ __forceinline__ bool chunk_exists(int c)
{
    using S = Stage<D, NW, 0>;
    return S::NCH % S::T == 0 || c < S::NCH;
}

template <int D, int NW, int KVF>
__device__ __forceinline__ void stage_pages(Stage<D, NW, KVF> &st, const RowAddr &ra, int k0,
                                            int tid)
{
    using S = Stage<D, NW, KVF>;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) st.page[i] = ra.page_id(k0 + (tid + i * S::T) / CPR);
}

// Global -> registers.  Keys past the request are clamped to its last key
// (a valid row); stage_store zeroes them, so no unwritten slot (whatever its
// bits, even NaN) ever reaches an MFMA.
template <int D, int NW, int KVF>
__device__ __forceinline__ void stage_load(Stage<D, NW, KVF> &st, const PrefillArgs &a,
                                           const RowAddr &ra, int k0, int tid)
{
    using S = Stage<D, NW, KVF>;
    using Raw = typename S::Raw;
    using Elem = typename std::conditional<KVF == 0, uint16_t, uint8_t>::type;
    constexpr int CPR = D / 8;
    const Elem *K = static_cast<const Elem *>(a.k);
    const Elem *V = static_cast<const Elem *>(a.v);
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
        const int c = tid + i * S::T;
        if (chunk_exists<D, NW>(c)) {
            const int key = k0 + c / CPR;
            if (KVF == 0 && ra.clamp_key(key) >= ra.split) {
                // a new token's row of the contiguous K/V (16-bit, like the cache)
                const int64_t off = int64_t(ra.clamp_key(key) + ra.ext_row0) * ra.slot_stride +
                                    ra.head_off + (c % CPR) * 8;
                st.k[i] = *reinterpret_cast<const Raw *>(static_cast<const Elem *>(a.k_ext) + off);
                st.v[i] = *reinterpret_cast<const Raw *>(static_cast<const Elem *>(a.v_ext) + off);
            } else {
                const int64_t off = ra.offset(st.page[i], key) + (c % CPR) * 8;
                st.k[i] = *reinterpret_cast<const Raw *>(K + off);
                st.v[i] = *reinterpret_cast<const Raw *>(V + off);
            }
        }
    }
}

// 16-bit bits of a staged chunk (8-bit caches: widened exactly, OCP e4m3 or
// e5m2 -> fp32 -> bf16 / half)
template <bool F16, int KVF>
__device__ __forceinline__ u32x4 chunk_bits(const typename Stage<64, 4, KVF>::Raw &raw)
{
    if constexpr (KVF == 0) return raw;
    else return __builtin_bit_cast(u32x4, widen_fp8<KVF, F16>(raw));
}

// Per-element window/causal/length mask of one 32-key tile for a lane's row
// (entry i: key k0 + 8*(i/4) + 4*hw + i%4).  Branch-free on purpose.
__device__ __forceinline__ void mask_tile(f32x16 &s, int k0, int hw, int p, int kv_len,
                                          int causal, int W)
{
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * hw + (i & 3);
        const bool vis = (key < kv_len) & ((causal == 0) | (key <= p)) & ((W < 0) | (key >= p - W));
        s[i] = vis ? s[i] : kNegInf;
    }
}

__device__ __forceinline__ float max16(const f32x16 &s)
{
    float a = fmaxf(s[0], fmaxf(s[1], s[2]));
    float b = fmaxf(s[3], fmaxf(s[4], s[5]));
    float c = fmaxf(s[6], fmaxf(s[7], s[8]));
    float d = fmaxf(s[9], fmaxf(s[10], s[11]));
    float e = fmaxf(s[12], fmaxf(s[13], s[14]));
    return fmaxf(fmaxf(a, fmaxf(b, c)), fmaxf(fmaxf(d, e), s[15]));
}

template <bool F16, int D, int NW, int KVF>
__device__ __forceinline__ void stage_store(Stage<D, NW, KVF> &st, PrefillBuf<D> &b, int k0,
                                            int kv_len, int tid)
{
    using S = Stage<D, NW, KVF>;
    constexpr int CPR = D / 8;
    if (k0 + KT > kv_len) {
        // the request's last tile: keys past its end become zeros
#pragma unroll
        for (int i = 0; i < S::KCH; ++i) {
            const bool past = k0 + (tid + i * S::T) / CPR >= kv_len;
            const typename S::Raw z = {};
            st.k[i] = past ? z : st.k[i];
            st.v[i] = past ? z : st.v[i];
        }
    }
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
        const int c = tid + i * S::T;
        if (chunk_exists<D, NW>(c)) {
            *reinterpret_cast<u32x4 *>(&b.k[c / CPR][(c % CPR) * 8]) = chunk_bits<F16, KVF>(st.k[i]);
            *reinterpret_cast<u32x4 *>(&b.v[c / CPR][(c % CPR) * 8]) = chunk_bits<F16, KVF>(st.v[i]);
        }
    }
}

// S^T[32 keys x 32 rows] = K . Q^T for the tile in b.
template <int D, bool F16>
__device__ __forceinline__ f32x16 qk_tile(const PrefillBuf<D> &b, const bf16x8 (&qf)[D / 16],
                                          int l32, int hw)
{
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&b.k[l32][ks * 16 + hw * 8]);
        s = mfma32x32x16<F16>(kf, qf[ks], s);
    }
    return s;
}

// O^T += V^T . P^T for one 32-key tile (two k-steps of 16 keys).
template <int D, bool F16>
__device__ __forceinline__ void pv_tile(const PrefillBuf<D> &b, const bf16x8 (&pb)[2],
                                        f32x16 (&o)[D / 32], int tr_key, int tr_dim)
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const uint16_t *v0 = &b.v[16 * kk + tr_key][32 * dt + tr_dim];
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)v0);
            const i16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v0 + 8 * (D + VPAD)));
            const bf16x8 va =
                __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[dt] = mfma32x32x16<F16>(va, pb[kk], o[dt]);
        }
}

// Direct-to-LDS staging (DMA = true, head_dim 128, 8 waves).  Each K/V row of
// a tile is fetched with one global_load_lds_dword: the 64 lanes move the
// row's 256 bytes straight into its padded LDS row, with no registers, no
// address arithmetic per lane (a scalar base per row plus the lane's fixed
// 4-byte offset) and no LDS store instruction.  The loads are tracked only
// by the vector memory counter, so the tile sets are waited for by hand: six
// tiles are in flight ahead of the one being computed, in eight LDS sets.
// The page ids of the item's key range sit in an LDS table filled by the
// item's prologue, so finding a row's page is an LDS read.
constexpr int DMA_SETS = 8;
constexpr int DMA_AHEAD = DMA_SETS - 2;  // sets j-1 (lagging PV) .. j+AHEAD
constexpr int DMA_ROWS = KT / 8;         // rows of K (and of V) per wave per tile
constexpr int DMA_PER_TILE = 2 * DMA_ROWS;  // loads per wave per tile

// s_waitcnt vmcnt(N), the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Row loads global -> LDS (global_load_lds_dword): the 64 lanes move one
// 256-byte row, lane i's bytes 4i..4i+3 to LDS byte address M0 + 4i.  M0 is
// a register the compiler reserves, so each statement restores it.
//
// One K row and the V row at the same offset:
__device__ __forceinline__ void dma_row_kv(uint32_t mk, uint32_t mv, uint32_t lane_off,
                                           const void *ksrc, const void *vsrc)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\tglobal_load_lds_dword %3, %4\n\t"
                 "s_mov_b32 m0, %2\n\tglobal_load_lds_dword %3, %5\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(mk), "s"(mv), "v"(lane_off), "s"(ksrc), "s"(vsrc)
                 : "memory");
}

// Four K rows and four V rows at the lane offsets off[0..3] from one base each:
__device__ __forceinline__ void dma_rows4_kv(const uint32_t (&mk)[4], const uint32_t (&mv)[4],
                                             const uint32_t (&off)[4], const void *kb,
                                             const void *vb)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\tglobal_load_lds_dword %9, %13\n\t"
                 "s_mov_b32 m0, %2\n\tglobal_load_lds_dword %10, %13\n\t"
                 "s_mov_b32 m0, %3\n\tglobal_load_lds_dword %11, %13\n\t"
                 "s_mov_b32 m0, %4\n\tglobal_load_lds_dword %12, %13\n\t"
                 "s_mov_b32 m0, %5\n\tglobal_load_lds_dword %9, %14\n\t"
                 "s_mov_b32 m0, %6\n\tglobal_load_lds_dword %10, %14\n\t"
                 "s_mov_b32 m0, %7\n\tglobal_load_lds_dword %11, %14\n\t"
                 "s_mov_b32 m0, %8\n\tglobal_load_lds_dword %12, %14\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(mk[0]), "s"(mk[1]), "s"(mk[2]), "s"(mk[3]), "s"(mv[0]), "s"(mv[1]),
                   "s"(mv[2]), "s"(mv[3]), "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]),
                   "s"(kb), "s"(vb)
                 : "memory");
}

// Key split: a row's partial over one key chunk -- o normalised over the
// chunk's keys (times v_scale), rounded to the query dtype, and its lse in
// fp32 (-inf when no key of the chunk is visible) -- to slot row sl of the
// float workspace.  Lane (l32, hw) holds dims 32 dt + 8 m0 + 4 hw + m1 of its
// row in o[dt][4 m0 + m1].
template <bool F16, int DT>
__device__ __forceinline__ void store_partial(const PrefillArgs &a, int64_t sl,
                                              const f32x16 (&o)[DT], float m, float l, int hw)
{
    const float w_self = l > 0.f ? a.v_scale / l : 0.f;
    uint16_t *PO = static_cast<uint16_t *>(a.part_o) + sl * (DT * 32);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int m0 = 0; m0 < 4; ++m0) {
            f32x4 v4;
#pragma unroll
            for (int m1 = 0; m1 < 4; ++m1) v4[m1] = o[dt][4 * m0 + m1] * w_self;
            *reinterpret_cast<bf16x4 *>(PO + dt * 32 + 8 * m0 + 4 * hw) = to16x4<F16>(v4);
        }
    if (hw == 0) a.part_lse[sl] = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
}

template <int D, int NW, bool DMA, bool F16, int KVF>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillArgs a)
{
    static_assert(!DMA || (D == 128 && NW == 8 && KVF == 0),
                  "direct-to-LDS staging: D = 128, 8 waves, 16-bit K/V");
    constexpr int KSTEPS = D / 16;  // QK k-steps
    constexpr int DT = D / 32;      // O^T dim tiles
    constexpr int NS = DMA ? DMA_SETS : NBUF;  // LDS tile sets (a power of two)
    struct Lds {
        PrefillBuf<D> set[NS];
        int32_t pages[DMA ? kPrefillDmaPages : 1];
    };
    __shared__ __attribute__((aligned(16))) Lds sh;
    PrefillBuf<D> *const lds = sh.set;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hw = lane >> 5;
    const int G = 1 << a.log2_group;
    const int n_items = a.ws[kHdrNumItems];
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    const int W = a.window_left;
    const float c = a.scale_log2;
    const float cap_a = a.cap_a;

    // transposing-read coordinates of this lane (see PrefillBuf)
    const int tr_key = 4 * hw + ((lane & 15) >> 2);             // + 16*kk (+8)
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32*dt

    RowAddr ra;
    ra.kv_indices = a.kv_indices;
    ra.num_pages = a.num_pages;
    ra.slot_stride = int64_t(a.num_kv_heads) * D;
    ra.page_stride = ra.slot_stride * a.page_rows;
    ra.log2_page = a.log2_page;
    ra.page_mask = a.page_size - 1;

    // direct-to-LDS staging: LDS byte address of set 0, the wave's rows
    const uint32_t lds0 =
        uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void *)lds));
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lane_off = 4u * uint32_t(lane);
    const uint32_t page_bytes = uint32_t(ra.page_stride * 2);
    const int32_t slot_bytes = int32_t(ra.slot_stride * 2);
    uint32_t row_off[DMA_ROWS];  // lane offset of row i of a same-page run
#pragma unroll
    for (int i = 0; i < DMA_ROWS; ++i) row_off[i] = lane_off + uint32_t(i * slot_bytes);
    const char *const Kb = static_cast<const char *>(a.k);
    const char *const Vb = static_cast<const char *>(a.v);

    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const int32_t *w = a.ws + kHeaderWords + int64_t(it) * kPrefillItemWords;
        const int hk = w[kPiKvHead], q_begin = w[kPiQBegin], q_count = w[kPiQCount];
        const int pos0 = w[kPiPos0], kv_len = w[kPiKvLen];
        const int kv_begin = w[kPiKvBegin];
        // (a key chunk of a split tile ends at a key tile boundary)
        const int kv_end = min(a.causal ? min(kv_len, pos0 + q_count) : kv_len, w[kPiKvEnd]);
        const int slot0 = w[kPiSlot], slot_stride = w[kPiSlotStride];
        const int pos_last = pos0 + q_count - 1;
        const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + KT - 1) / KT : 0;
        ra.page_base = w[kPiPageBase];
        ra.kv_len = kv_len;
        ra.head_off = int64_t(hk) * D;
        ra.split = DMA ? INT32_MAX : w[kPiSplit];
        ra.ext_row0 = q_begin - pos0;
        const int pt_lo = kv_begin >> a.log2_page;
        const int32_t head_bytes = int32_t(ra.head_off * 2);

        // this lane's row (S^T and O^T keep one row per lane: column l32)
        const int row = wave * 32 + l32;
        const int row_tok = row >> a.log2_group, row_head = row & (G - 1);
        const bool row_valid = row_tok < q_count;
        const int p_row = pos0 + row_tok;
        const int64_t qrow =
            (int64_t(q_begin + row_tok) * a.num_qo_heads + hk * G + row_head) * D;

        bf16x8 qf[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            qf[ks] = row_valid ? load_bf16x8(Q + qrow + ks * 16 + hw * 8) : zero_bf16x8();

        float m = kNegInf, l = 0.f;
        f32x16 o[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

        // Issue the row loads of tile t (direct-to-LDS staging): the wave's
        // DMA_ROWS consecutive rows of K and of V.  Keys past the item's last
        // tile or past the request read its last loaded key (finite data,
        // masked out), so tiles past the end can be issued as well and every
        // wave always has the same number of loads in flight.  Page ids come
        // from the LDS table; `pg0` is the id of the page of the first row.
        const int kv_last = min(kv_begin + ntiles * KT, kv_len) - 1;
        // page id of `key` from the LDS table; the planner keeps every index
        // inside the entries the prologue wrote, the clamps only keep a
        // corrupt work list from reading past the table or the cache
        auto page_entry = [&](int key) __attribute__((always_inline)) {
            const int e = min(max((key >> a.log2_page) - pt_lo, 0), kPrefillDmaPages - 1);
            return min(max(sh.pages[e], 0), int32_t(a.num_pages - 1));
        };
        auto dma_tile = [&](int t, int32_t pg0) __attribute__((always_inline)) {
            const int k0 = kv_begin + t * KT;
            const int r0 = DMA_ROWS * uwave;
            const uint32_t set_b = lds0 + uint32_t((t & (NS - 1)) * sizeof(PrefillBuf<D>));
            const uint32_t mk = set_b + uint32_t(offsetof(PrefillBuf<D>, k) + r0 * (D + KPAD) * 2);
            const uint32_t mv = set_b + uint32_t(offsetof(PrefillBuf<D>, v) + r0 * (D + VPAD) * 2);
            const int key0 = min(k0 + r0, kv_last);
            static_assert(DMA_ROWS == 4, "dma_rows4_kv moves four rows");
            if (k0 + r0 + DMA_ROWS - 1 <= kv_last &&
                (key0 & ra.page_mask) + DMA_ROWS <= a.page_size) {
                // the rows are consecutive slots of one page: one scalar base,
                // the row step sits in the lane offsets
                const int64_t off = int64_t(uint64_t(uint32_t(pg0)) * page_bytes) +
                                    int32_t((key0 & ra.page_mask) * slot_bytes + head_bytes);
                uint32_t m0k[DMA_ROWS], m0v[DMA_ROWS];
#pragma unroll
                for (int i = 0; i < DMA_ROWS; ++i) {
                    m0k[i] = mk + uint32_t(i * (D + KPAD) * 2);
                    m0v[i] = mv + uint32_t(i * (D + VPAD) * 2);
                }
                dma_rows4_kv(m0k, m0v, row_off, Kb + off, Vb + off);
            } else {
#pragma unroll
                for (int i = 0; i < DMA_ROWS; ++i) {
                    const int key = min(k0 + r0 + i, kv_last);
                    const int32_t pg = __builtin_amdgcn_readfirstlane(page_entry(key));
                    const int64_t off = int64_t(uint64_t(uint32_t(pg)) * page_bytes) +
                                        int32_t((key & ra.page_mask) * slot_bytes + head_bytes);
                    dma_row_kv(mk + uint32_t(i * (D + KPAD) * 2), mv + uint32_t(i * (D + VPAD) * 2),
                               lane_off, Kb + off, Vb + off);
                }
            }
        };
        // LDS read of the page id of the wave's first row of tile t
        auto dma_page = [&](int t) __attribute__((always_inline)) {
            return page_entry(min(kv_begin + t * KT + DMA_ROWS * uwave, kv_last));
        };

        Stage<D, NW, KVF> st;
        if constexpr (DMA) {
            // prologue: page table of the item (ids clamped into the cache),
            // then tiles 0 .. AHEAD-1 in flight; wait for tiles 0 and 1
            const int pt_n =
                ntiles > 0 ? min((kv_last >> a.log2_page) - pt_lo + 1, kPrefillDmaPages) : 0;
            for (int e = tid; e < pt_n; e += NW * 64) {
                const int32_t pg = a.kv_indices[ra.page_base + pt_lo + e];
                sh.pages[e] = min(max(pg, 0), int32_t(a.num_pages - 1));
            }
            // the Q operand and the page ids have landed (and nothing else is
            // in flight): later waits count only row loads
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (ntiles > 0) {
#pragma unroll 1
                for (int t = 0; t < DMA_AHEAD; ++t)
                    dma_tile(t, __builtin_amdgcn_readfirstlane(dma_page(t)));
                wait_vmcnt<(DMA_AHEAD - 2) * DMA_PER_TILE>();  // tiles 0 and 1 landed
            }
            __syncthreads();
        } else {
            // prologue: tiles 0 and 1 in LDS sets 0 and 1, tile 2 in registers,
            // tile 3's page ids read
            if (ntiles > 0) {
                stage_pages(st, ra, kv_begin, tid);
                stage_load(st, a, ra, kv_begin, tid);
                stage_pages(st, ra, kv_begin + KT, tid);
                stage_store<F16>(st, lds[0], kv_begin, kv_len, tid);
                if (ntiles > 1) {
                    stage_load(st, a, ra, kv_begin + KT, tid);
                    stage_pages(st, ra, kv_begin + 2 * KT, tid);
                    stage_store<F16>(st, lds[1], kv_begin + KT, kv_len, tid);
                    if (ntiles > 2) {
                        stage_load(st, a, ra, kv_begin + 2 * KT, tid);
                        stage_pages(st, ra, kv_begin + 3 * KT, tid);
                    }
                }
            }
            __syncthreads();
            // Everything issued so far (the Q operand included) has landed: say
            // so once here, so the loop's first MFMA does not wait for the
            // in-flight K/V loads of later tiles.
            __builtin_amdgcn_s_waitcnt(0);
        }
        // S^T of tile 0 (s_a); each step leaves the next tile's in s_b
        f32x16 s_a, s_b;
        if (ntiles > 0) s_a = qk_tile<D, F16>(lds[0], qf, l32, hw);

        // Ping-pong: with 8 waves, waves w and w+4 share a SIMD.  Waves 4..7
        // issue the PV product of a tile one iteration late, so in every
        // iteration one wave of each SIMD starts with its exponentials
        // (vector ALU) while the other starts with PV (matrix core).
        const bool lag = NW == 8 && uwave >= 4;
        bf16x8 pb_a[2] = {zero_bf16x8(), zero_bf16x8()};
        bf16x8 pb_b[2] = {zero_bf16x8(), zero_bf16x8()};

        // one key tile: s_in = S^T of tile j in, s_out = S^T of tile j+1 out;
        // pb_out = P^T of tile j, pb_in = P^T of tile j-1 (lagging waves)
        auto step = [&](int j, const f32x16 &s_in, f32x16 &s_out, bf16x8 (&pb_out)[2],
                        const bf16x8 (&pb_in)[2]) __attribute__((always_inline)) {
            const int k0 = kv_begin + j * KT;
            // page of tile j+AHEAD, requested early (used at the end of the step)
            int32_t pg_next = 0;
            if constexpr (DMA) pg_next = dma_page(j + DMA_AHEAD);
            if (lag && j > 0) pv_tile<D, F16>(lds[(j - 1) & (NS - 1)], pb_in, o, tr_key, tr_dim);
            // K operands of tile j+1 (its LDS set is ready; after the last tile
            // they are read but unused), requested before the row maximum
            const PrefillBuf<D> &bn = lds[(j + 1) & (NS - 1)];
            bf16x8 kf[KSTEPS];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                kf[ks] = *reinterpret_cast<const bf16x8 *>(&bn.k[l32][ks * 16 + hw * 8]);

            // accumulator entry i holds key k0 + 8*(i/4) + 4*hw + i%4 of this row
            f32x16 s = s_in;
            if (cap_a != 0.f) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = soft_cap_unit(s[i], cap_a);
            }
            const bool interior = k0 + KT <= kv_len && (!a.causal || k0 + KT - 1 <= pos0) &&
                                  (W < 0 || k0 >= pos_last - W);
            if (!interior) mask_tile(s, k0, hw, p_row, kv_len, a.causal, W);
            // row maximum: lane-local over 16 keys, then across the two halves
            // of the wave with a lane swap (a VALU op, no LDS round trip)
            float mx = max16(s);
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                                 __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
            }

            // lazy rescale: keep the running maximum unless some row's grows by
            // more than 2^8 (probabilities then stay below 2^8, exact in fp32
            // and in bf16 range), so most tiles skip the O rescale.  O holds PV
            // up to tile j-1 here, for both wave groups.
            if (__any(mx > m + kRescaleLog2)) {
                const float m_new = fmaxf(m, mx);
                const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m - m_new);
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
                m = m_new;
            }
            const float mu = m == kNegInf ? 0.f : m;

            // S^T of tile j+1 interleaved by hand with this tile's exponentials:
            // each dependent QK MFMA is followed by the FMA+exp of 16/KSTEPS
            // scores, which the vector ALU runs while the matrix core works.
            // The fences keep the compiler from regrouping them.
            constexpr int EPS = 16 / KSTEPS;  // scores per QK step (D=128: 2)
#pragma unroll
            for (int i = 0; i < 16; ++i) s_out[i] = 0.f;
            f32x16 pr;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                s_out = mfma32x32x16<F16>(kf[ks], qf[ks], s_out);
#pragma unroll
                for (int e = 0; e < EPS; ++e) {
                    const int i = ks * EPS + e;
                    pr[i] = fast_exp2(__builtin_fmaf(s[i], c, -mu));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // row sum as a tree (short dependency chains)
            float t8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t8[i] = pr[2 * i] + pr[2 * i + 1];
            l += ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                f32x8 p8;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) p8[jj] = pr[8 * kk + jj];
                pb_out[kk] = to16x8<F16>(p8);
            }
            if (!lag) pv_tile<D, F16>(lds[j & (NS - 1)], pb_out, o, tr_key, tr_dim);

            if constexpr (DMA) {
                // tile j+AHEAD into the set tile j-2 used; then tile j+2 must
                // have landed (in every wave) before the barrier
                dma_tile(j + DMA_AHEAD, __builtin_amdgcn_readfirstlane(pg_next));
                wait_vmcnt<(DMA_AHEAD - 2) * DMA_PER_TILE>();
            } else {
                // stage tile j+2 into the free LDS set, start loading tile j+3
                if (j + 2 < ntiles) {
                    stage_store<F16>(st, lds[(j + 2) & (NS - 1)], k0 + 2 * KT, kv_len, tid);
                    if (j + 3 < ntiles) {
                        stage_load(st, a, ra, k0 + 3 * KT, tid);
                        stage_pages(st, ra, k0 + 4 * KT, tid);
                    }
                }
            }
            __syncthreads();
        };

        for (int j = 0; j < ntiles; ++j) {
            step(j, s_a, s_b, pb_a, pb_b);
            s_a = s_b;
            pb_b[0] = pb_a[0];
            pb_b[1] = pb_a[1];
        }
        if (lag && ntiles > 0) pv_tile<D, F16>(lds[(ntiles - 1) & (NS - 1)], pb_b, o, tr_key, tr_dim);

        // epilogue: the two half-waves hold disjoint keys of each row
        l += __shfl_xor(l, 32);
        if (row_valid && slot0 >= 0) {
            // one key chunk of a split tile: the row's partial to its slot
            store_partial<F16>(a, int64_t(slot0 + row_tok * slot_stride) * G + row_head, o, m, l,
                               hw);
        } else if (row_valid) {
            const int64_t lrow = int64_t(q_begin + row_tok) * a.num_qo_heads + hk * G + row_head;
            float w_self = l > 0.f ? a.v_scale / l : 0.f, w_other = 0.f;
            float lse_row = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
            if (a.fold_lse) {
                const Fold f = fold_weights(lse_row, a.fold_lse[lrow]);
                w_self *= f.self;
                w_other = f.other;
                lse_row = f.lse;
            }
            uint16_t *O = static_cast<uint16_t *>(a.o);
            const uint16_t *FO = static_cast<const uint16_t *>(a.fold_o);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int m0 = 0; m0 < 4; ++m0) {
                    const int64_t at = qrow + dt * 32 + 8 * m0 + 4 * hw;
                    f32x4 v4;
#pragma unroll
                    for (int m1 = 0; m1 < 4; ++m1) v4[m1] = o[dt][4 * m0 + m1] * w_self;
                    if (FO) {
                        const f32x4 f4 = from16x4<F16>(*reinterpret_cast<const bf16x4 *>(FO + at));
#pragma unroll
                        for (int m1 = 0; m1 < 4; ++m1) v4[m1] += f4[m1] * w_other;
                    }
                    *reinterpret_cast<bf16x4 *>(O + at) = to16x4<F16>(v4);
                }
            if (a.lse && hw == 0) a.lse[lrow] = lse_row;
        }
        __syncthreads();  // the next item's prologue overwrites the LDS sets
    }
}

// Wide variant for head_dim <= 128: 4 waves x 64 rows (two 32-row N tiles per
// wave, 256 rows per workgroup), one wave per SIMD.  Every K / V^T operand
// read from LDS feeds two MFMAs (half the LDS traffic of the 32-row waves),
// and the wave pipelines its own work: iteration j issues the PV MFMAs of
// tile j-1 and the QK MFMAs of tile j+1 -- neither depends on tile j's
// softmax -- interleaved instruction by instruction with tile j's max and
// exponentials, so the matrix cores and the vector ALUs run together.  Four
// LDS tile sets are live: V of j-1, V of j, K and V of j+1, and j+2 being
// written.  A rescale of O (rare, see kRescaleLog2) is applied after PV of
// tile j-1 has landed, before PV of tile j.
constexpr int WIDE_SETS = 4;

template <int D>
struct WideOps {
    static constexpr int KS = D / 16;  // QK k-steps
    static constexpr int DT = D / 32;  // O^T dim tiles
    static constexpr int NQ = 2 * DT;  // V^T operands per tile (dim tile x 16-key step)
};

template <int D>
__device__ __forceinline__ bf16x8 wide_vop(const PrefillBuf<D> &b, int q, int tr_key, int tr_dim)
{
    const int dt = q >> 1, kk = q & 1;
    const uint16_t *v0 = &b.v[16 * kk + tr_key][32 * dt + tr_dim];
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)v0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(v0 + 8 * (D + VPAD)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D>
__device__ __forceinline__ bf16x8 wide_kop(const PrefillBuf<D> &b, int ks, int l32, int hw)
{
    return *reinterpret_cast<const bf16x8 *>(&b.k[l32][ks * 16 + hw * 8]);
}

template <int D, bool F16>
__global__ __launch_bounds__(256) void prefill_wide_kernel(PrefillArgs a)
{
    constexpr int KS = WideOps<D>::KS, DT = WideOps<D>::DT, NQ = WideOps<D>::NQ;
    constexpr int NW = 4;
    __shared__ __attribute__((aligned(16))) PrefillBuf<D> lds[WIDE_SETS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hw = lane >> 5;
    const int G = 1 << a.log2_group;
    const int n_items = a.ws[kHdrNumItems];
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    const int W = a.window_left;
    const float c = a.scale_log2;
    const int tr_key = 4 * hw + ((lane & 15) >> 2);
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    RowAddr ra;
    ra.kv_indices = a.kv_indices;
    ra.num_pages = a.num_pages;
    ra.slot_stride = int64_t(a.num_kv_heads) * D;
    ra.page_stride = ra.slot_stride * a.page_rows;
    ra.log2_page = a.log2_page;
    ra.page_mask = a.page_size - 1;

    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const int32_t *w = a.ws + kHeaderWords + int64_t(it) * kPrefillItemWords;
        const int hk = w[kPiKvHead], q_begin = w[kPiQBegin], q_count = w[kPiQCount];
        const int pos0 = w[kPiPos0], kv_len = w[kPiKvLen];
        const int kv_begin = w[kPiKvBegin];
        const int kv_end = a.causal ? min(kv_len, pos0 + q_count) : kv_len;
        const int pos_last = pos0 + q_count - 1;
        const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + KT - 1) / KT : 0;
        ra.page_base = w[kPiPageBase];
        ra.kv_len = kv_len;
        ra.head_off = int64_t(hk) * D;

        // the lane's two rows: N tile n holds row wave*64 + 32n + l32
        int row_tok[2], row_head[2], p_row[2];
        bool row_valid[2];
        int64_t qrow[2];
        bf16x8 qf[2][KS];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int row = wave * 64 + 32 * n + l32;
            row_tok[n] = row >> a.log2_group;
            row_head[n] = row & (G - 1);
            row_valid[n] = row_tok[n] < q_count;
            p_row[n] = pos0 + row_tok[n];
            qrow[n] = (int64_t(q_begin + row_tok[n]) * a.num_qo_heads + hk * G + row_head[n]) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[n][ks] = row_valid[n] ? load_bf16x8(Q + qrow[n] + ks * 16 + hw * 8)
                                         : zero_bf16x8();
        }

        float m[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
        f32x16 o[2][DT];
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[n][dt][i] = 0.f;

        // prologue: tiles 0 and 1 in sets 0 and 1, tile 2 in registers, tile 3's
        // page ids read; the V rows of set 3 (read as "tile -1") are zeroed
        Stage<D, NW, 0> st;
        for (int e = tid; e < KT * (D + VPAD) / 8; e += NW * 64)
            reinterpret_cast<u32x4 *>(&lds[WIDE_SETS - 1].v[0][0])[e] = u32x4{0u, 0u, 0u, 0u};
        if (ntiles > 0) {
            stage_pages(st, ra, kv_begin, tid);
            stage_load(st, a, ra, kv_begin, tid);
            stage_pages(st, ra, kv_begin + KT, tid);
            stage_store<F16>(st, lds[0], kv_begin, kv_len, tid);
            if (ntiles > 1) {
                stage_load(st, a, ra, kv_begin + KT, tid);
                stage_pages(st, ra, kv_begin + 2 * KT, tid);
                stage_store<F16>(st, lds[1], kv_begin + KT, kv_len, tid);
                if (ntiles > 2) {
                    stage_load(st, a, ra, kv_begin + 2 * KT, tid);
                    stage_pages(st, ra, kv_begin + 3 * KT, tid);
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_s_waitcnt(0);

        f32x16 s_cur[2];
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) s_cur[n][i] = 0.f;
        if (ntiles > 0) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kf = wide_kop<D>(lds[0], ks, l32, hw);
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    s_cur[n] = mfma32x32x16<F16>(kf, qf[n][ks], s_cur[n]);
            }
        }
        bf16x8 p_prev[2][2];
#pragma unroll
        for (int n = 0; n < 2; ++n) p_prev[n][0] = p_prev[n][1] = zero_bf16x8();

        for (int j = 0; j < ntiles; ++j) {
            const int k0 = kv_begin + j * KT;
            const int cur = j & 3, nxt = (j + 1) & 3, nn = (j + 2) & 3, prv = (j + 3) & 3;

            // exact mask on tiles that straddle the window edge, the diagonal or
            // the end of the keys (entry i: key k0 + 8*(i/4) + 4*hw + i%4)
            const bool interior = k0 + KT <= kv_len && (!a.causal || k0 + KT - 1 <= pos0) &&
                                  (W < 0 || k0 >= pos_last - W);
            if (a.cap_a != 0.f) {
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int i = 0; i < 16; ++i) s_cur[n][i] = soft_cap_unit(s_cur[n][i], a.cap_a);
            }
            if (!interior) {
#pragma unroll
                for (int n = 0; n < 2; ++n) mask_tile(s_cur[n], k0, hw, p_row[n], kv_len, a.causal, W);
            }

            // region 1: PV of tile j-1 on the matrix cores, row maxima on the VALU
            float mx[2] = {kNegInf, kNegInf};
            {
                const PrefillBuf<D> &bp = lds[prv];
                bf16x8 va = wide_vop<D>(bp, 0, tr_key, tr_dim);
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const bf16x8 vc = va;
                    if (q + 1 < NQ) va = wide_vop<D>(bp, q + 1, tr_key, tr_dim);
                    const int dt = q >> 1, kk = q & 1;
#pragma unroll
                    for (int n = 0; n < 2; ++n)
                        o[n][dt] = mfma32x32x16<F16>(vc, p_prev[n][kk], o[n][dt]);
                    // 32 scores over NQ steps
#pragma unroll
                    for (int e = 0; e < 32 / NQ; e += 2) {
                        const int f = q * (32 / NQ) + e, n = f >> 4, i = f & 15;
                        mx[n] = fmaxf(mx[n], fmaxf(s_cur[n][i], s_cur[n][i + 1]));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            float m_new[2], alpha[2], mu[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) mx[n] = fmaxf(mx[n], __shfl_xor(mx[n], 32)) * c;
            const bool need = __any(mx[0] > m[0] + kRescaleLog2 || mx[1] > m[1] + kRescaleLog2);
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                m_new[n] = need ? fmaxf(m[n], mx[n]) : m[n];
                alpha[n] = m_new[n] == kNegInf ? 1.f : fast_exp2(m[n] - m_new[n]);
                mu[n] = m_new[n] == kNegInf ? 0.f : m_new[n];
            }

            // region 2: QK of tile j+1 (after the last tile the result is unused)
            // on the matrix cores, exponentials of tile j on the VALU, packed to
            // bf16 pairs as they are made
            f32x16 s_nxt[2];
            bf16x8 p_cur[2][2];
            float rs[2] = {0.f, 0.f};
            {
                const PrefillBuf<D> &bn = lds[nxt];
                bf16x8 kf = wide_kop<D>(bn, 0, l32, hw);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 kc = kf;
                    if (ks + 1 < KS) kf = wide_kop<D>(bn, ks + 1, l32, hw);
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        if (ks == 0) {
                            const f32x16 z = {};
                            s_nxt[n] = mfma32x32x16<F16>(kc, qf[n][0], z);
                        } else {
                            s_nxt[n] = mfma32x32x16<F16>(kc, qf[n][ks], s_nxt[n]);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 32 / KS; e += 2) {
                        const int f = ks * (32 / KS) + e, n = f >> 4, i = f & 15;
                        const float e0 = fast_exp2(__builtin_fmaf(s_cur[n][i], c, -mu[n]));
                        const float e1 = fast_exp2(__builtin_fmaf(s_cur[n][i + 1], c, -mu[n]));
                        rs[n] += e0 + e1;
                        const bf16x2 pk = to16x2<F16>(f32x2{e0, e1});
                        p_cur[n][i >> 3][i & 7] = pk[0];
                        p_cur[n][i >> 3][(i & 7) + 1] = pk[1];
                        // keep this step's VALU work here, between its MFMAs
                        asm volatile("" ::"v"(rs[n]));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) l[n] = l[n] * alpha[n] + rs[n];
            if (need) {
                // O holds PV up to tile j-1 at the old maximum
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) o[n][dt] *= alpha[n];
            }

            // stage tile j+2 into its LDS set, start loading tile j+3
            if (j + 2 < ntiles) {
                stage_store<F16>(st, lds[nn], k0 + 2 * KT, kv_len, tid);
                if (j + 3 < ntiles) {
                    stage_load(st, a, ra, k0 + 3 * KT, tid);
                    stage_pages(st, ra, k0 + 4 * KT, tid);
                }
            }
            __syncthreads();
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                s_cur[n] = s_nxt[n];
                p_prev[n][0] = p_cur[n][0];
                p_prev[n][1] = p_cur[n][1];
                m[n] = m_new[n];
            }
        }

        // epilogue: PV of the last tile, then normalise
        if (ntiles > 0) {
            const PrefillBuf<D> &bl = lds[(ntiles - 1) & 3];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const bf16x8 vc = wide_vop<D>(bl, q, tr_key, tr_dim);
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    o[n][q >> 1] = mfma32x32x16<F16>(vc, p_prev[n][q & 1], o[n][q >> 1]);
            }
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            float ln = l[n] + __shfl_xor(l[n], 32);
            if (row_valid[n]) {
                const int64_t lrow =
                    int64_t(q_begin + row_tok[n]) * a.num_qo_heads + hk * G + row_head[n];
                float w_self = ln > 0.f ? a.v_scale / ln : 0.f, w_other = 0.f;
                float lse_row = ln > 0.f ? (m[n] + fast_log2(ln)) * kLn2 : kNegInf;
                if (a.fold_lse) {
                    const Fold f = fold_weights(lse_row, a.fold_lse[lrow]);
                    w_self *= f.self;
                    w_other = f.other;
                    lse_row = f.lse;
                }
                uint16_t *O = static_cast<uint16_t *>(a.o);
                const uint16_t *FO = static_cast<const uint16_t *>(a.fold_o);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int m0 = 0; m0 < 4; ++m0) {
                        const int64_t at = qrow[n] + dt * 32 + 8 * m0 + 4 * hw;
                        f32x4 v4;
#pragma unroll
                        for (int m1 = 0; m1 < 4; ++m1) v4[m1] = o[n][dt][4 * m0 + m1] * w_self;
                        if (FO) {
                            const f32x4 f4 = from16x4<F16>(*reinterpret_cast<const bf16x4 *>(FO + at));
#pragma unroll
                            for (int m1 = 0; m1 < 4; ++m1) v4[m1] += f4[m1] * w_other;
                        }
                        *reinterpret_cast<bf16x4 *>(O + at) = to16x4<F16>(v4);
                    }
                if (a.lse && hw == 0) a.lse[lrow] = lse_row;
            }
        }
        __syncthreads();  // the next item's prologue overwrites the LDS sets
    }
}

// 64-key steps with 16-byte direct-to-LDS loads (variant 5: head_dim 128,
// 8 waves x 32 rows, 16-bit K/V).
//
// Each step covers a 64-key tile as two 32-key halves, so a wave's S^T of
// the next tile is two independent MFMA chains (one per half) and the row
// maximum, the lazy-rescale test, the page-id read, the load issue and the
// barrier are paid once per 64 keys.  The iteration for tile j runs four
// quarters (half h, 16-key step kk); each quarter issues four MFMAs of
// S^T(j+1), makes the next quarter's probabilities on the vector ALU and
// issues the four O^T += V^T.P^T MFMAs of its own 16 keys.
//
// Staging.  A K or V tile is 64 rows of 256 bytes stored unpadded; one
// global_load_lds_dwordx4 moves four rows (lane i writes LDS bytes
// 16i..16i+15 of the 1 KiB block), so a wave stages its 8 K rows and 8 V
// rows of a tile with four instructions from one scalar base when the 8 keys
// share a page.  Each lane may fetch any 16-byte chunk of the four rows, so
// the chunks are placed within a block to suit the operand reads: no two
// lanes of a read group share a bank position, and the four reads of a
// quarter lie 256 bytes apart (one lane base plus immediate offsets).  K and
// V tiles sit in two three-tile rings, so with the loop unrolled by three
// every ring position is a compile-time constant.
constexpr int BIG_T = 64;                     // keys per step
constexpr int BIG_ROW = 256;                  // bytes per K / V row
constexpr int BIG_HALF = BIG_T * BIG_ROW;     // K (or V) bytes of one tile

// Four 16-byte row-group loads from one scalar base per tensor: K rows to
// LDS mk and mk + 1024 (lane offsets dk0, dk1), V rows to mv and mv + 1024
// (dv0, dv1).  M0 holds the LDS destination and is restored afterwards.
__device__ __forceinline__ void big_dma4(uint32_t mk, uint32_t mv, uint32_t dk0, uint32_t dk1,
                                         uint32_t dv0, uint32_t dv1, const void *kb,
                                         const void *vb)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %5, %9\n\t"
                 "s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %6, %9\n\t"
                 "s_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %7, %10\n\t"
                 "s_mov_b32 m0, %4\n\tglobal_load_lds_dwordx4 %8, %10\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(mk), "s"(mk + 1024u), "s"(mv), "s"(mv + 1024u), "v"(dk0), "v"(dk1),
                   "v"(dv0), "v"(dv1), "s"(kb), "s"(vb)
                 : "memory");
}

// One 16-byte row-group load with a per-lane 64-bit address.
__device__ __forceinline__ void big_dma1(uint32_t m, const void *src)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(m), "v"(src)
                 : "memory");
}

// A wave-uniform value the optimiser must treat as unknown (kept in an SGPR).
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t x)
{
    asm volatile("" : "+s"(x));
    return x;
}

__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>(
        static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ i16x4 lds_tr(uint32_t addr)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_i16x4 *>(static_cast<uintptr_t>(addr)));
}

template <bool F16>
__global__ __launch_bounds__(512) void prefill_big_kernel(PrefillArgs a)
{
    constexpr int D = 128, KS = D / 16, DT = D / 32;
    struct Lds {
        uint8_t kset[3][BIG_HALF];  // K ring: tile t in kset[t % 3]
        uint8_t vset[3][BIG_HALF];  // V ring: tile t in vset[t % 3]
        int32_t pages[kPrefillBigPages];
        int32_t next_item;
    };
    __shared__ __attribute__((aligned(1024))) Lds sh;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hw = lane >> 5;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int G = 1 << a.log2_group;
    const int n_items = a.ws[kHdrNumItems];
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    const int W = a.window_left;
    const float c = a.scale_log2;
    const float cap_a = a.cap_a;

    const uint32_t lds_sets =
        uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void *)sh.kset));
    const uint32_t lds_v = lds_sets + uint32_t(3 * BIG_HALF);
    // LDS layout of a K or V tile: 1 KiB blocks of four rows; the 16-byte
    // chunk c (dims 8c..8c+7) of row R sits at position
    //   K: 16 (c / 4) + 4 ((c % 4 + R / 4) % 4) + R % 4
    //   V: 16 (c / 4) + 4 (R % 4) + c % 4
    // of block R / 4.  A 16-lane group of K operand reads (rows R..R+15, one
    // chunk) and a 32-lane group of V transposing reads (rows 4hw..4hw+3,
    // four chunks) then cover 16 distinct 16-byte bank positions, and the
    // four reads of a quarter (K: chunks c, c+4, c+8, c+12; V: dim tiles 0-3)
    // lie 256 bytes apart, so every operand address is a lane base plus an
    // immediate offset.
    // K operand of lane (l32, hw), k-step kk + 2u of half h: row 32h + l32,
    // chunk 4u + 2kk + hw.
    const uint32_t kvar0 = lds_sets + uint32_t(1024 * (l32 >> 2) + 16 * (l32 & 3) +
                                               64 * ((hw + (l32 >> 2)) & 3));
    const uint32_t kvar1 = lds_sets + uint32_t(1024 * (l32 >> 2) + 16 * (l32 & 3) +
                                               64 * ((2 + hw + (l32 >> 2)) & 3));
    // V^T transposing read of lane (hw, e, s16, q): row 4hw + e (+ 16kk, + 8,
    // + 32h), dims 32dt + 16s16 + 4q
    const uint32_t vvar = [&] {
        const int e = (lane & 15) >> 2, q = lane & 3, s16 = (lane >> 4) & 1;
        return lds_v + uint32_t(1024 * hw + 64 * e + 16 * (2 * s16 + (q >> 1)) + 8 * (q & 1));
    }();
    // staging: load i of a wave's rows 8 wave + 4i .. + 3 (block b = 2 wave + i)
    // writes LDS byte 16L of the block from lane L, which fetches
    //   K: row L % 4, chunk 4 (L / 16) + ((L / 4 - b) % 4)
    //   V: row (L / 4) % 4, chunk 4 (L / 16) + L % 4
    const int64_t slot_stride = int64_t(a.num_kv_heads) * D;
    const int32_t slot_bytes = int32_t(slot_stride * 2);
    const uint32_t page_bytes = uint32_t(slot_stride * a.page_rows * 2);
    const int kr = lane & 3, vr = (lane >> 2) & 3;
    const uint32_t kc0 = uint32_t(16 * (4 * (lane >> 4) + (((lane >> 2) - 2 * (wave & 1)) & 3)));
    const uint32_t kc1 = uint32_t(16 * (4 * (lane >> 4) + (((lane >> 2) - 2 * (wave & 1) - 1) & 3)));
    const uint32_t vc = uint32_t(16 * (4 * (lane >> 4) + (lane & 3)));
    const uint32_t row4 = uint32_t(4 * slot_bytes);
    const uint32_t dk0 = uint32_t(kr * slot_bytes) + kc0;
    const uint32_t dk1 = uint32_t(kr * slot_bytes) + row4 + kc1;
    const uint32_t dv0 = uint32_t(vr * slot_bytes) + vc;
    const uint32_t dv1 = dv0 + row4;
    const char *const Kb = static_cast<const char *>(a.k);
    const char *const Vb = static_cast<const char *>(a.v);
    const char *const Ke = static_cast<const char *>(a.k_ext);
    const char *const Ve = static_cast<const char *>(a.v_ext);
    const int page_mask = a.page_size - 1;

    // Items are handed out at run time, per XCD: item i belongs to XCD
    // i mod kXcds, where the grid-stride order would have run it, so items
    // that share key tiles (the same kv head, neighbouring query tiles) keep
    // sharing that XCD's L2.  Each workgroup starts with item blockIdx.x,
    // claims its XCD's next item from a counter in the workspace header as
    // it starts one, and learns it through LDS at the item's end, so
    // workgroups that run faster take more items.
    int32_t *const ctr = a.ws;
    const int xcd = blockIdx.x % kXcds;
    const int xcd_groups = (int(gridDim.x) - xcd + kXcds - 1) / kXcds;
    // Workgroups past the item count have nothing to claim: they leave without
    // touching the counters.
    if (int(blockIdx.x) >= n_items) return;
    // With a workgroup for every item nothing is handed out and the counters
    // are not touched.  Otherwise each processed item starts with one claim
    // on its XCD's counter, so that counter sees exactly as many claims as
    // the XCD has items, returning 0 .. n-1: the workgroup that draws n-1
    // makes its last claim and puts it back to 0 for the next launch.
    const bool claiming = int(gridDim.x) < n_items;
    const int xcd_items = (n_items - xcd + kXcds - 1) / kXcds;
    for (int it = blockIdx.x; it < n_items;) {
        int claimed = 0;
        if (claiming && tid == 0) {
            claimed = atomicAdd(ctr + kHdrNextItem + xcd, 1);
            if (claimed == xcd_items - 1) ctr[kHdrNextItem + xcd] = 0;
        }
        const int32_t *w = a.ws + kHeaderWords + int64_t(it) * kPrefillItemWords;
        const int hk = w[kPiKvHead], q_begin = w[kPiQBegin], q_count = w[kPiQCount];
        const int pos0 = w[kPiPos0], kv_len = w[kPiKvLen];
        const int kv_begin = w[kPiKvBegin];
        const int page_base = w[kPiPageBase];
        // one-pass cascade: keys from `split` on are the new tokens' rows
        const int split = w[kPiSplit];
        const int ext_row0 = q_begin - pos0;
        // (a key chunk of a split tile ends at a key tile boundary)
        const int kv_end = min(a.causal ? min(kv_len, pos0 + q_count) : kv_len, w[kPiKvEnd]);
        const int pos_last = pos0 + q_count - 1;
        const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + BIG_T - 1) / BIG_T : 0;
        const int pt_lo = kv_begin >> a.log2_page;
        const int32_t head_bytes = int32_t(hk * D * 2);
        // keys loaded past the item's tiles or the request read its last key
        const int kv_last = min(kv_begin + ntiles * BIG_T, kv_len) - 1;

        const int row = wave * 32 + l32;
        const int row_tok = row >> a.log2_group, row_head = row & (G - 1);
        const bool row_valid = row_tok < q_count;
        const int p_row = pos0 + row_tok;
        const int64_t qrow = (int64_t(q_begin + row_tok) * a.num_qo_heads + hk * G + row_head) * D;
        bf16x8 qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = row_valid ? load_bf16x8(Q + qrow + ks * 16 + hw * 8) : zero_bf16x8();

        float m = kNegInf, l = 0.f;
        f32x16 o[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

        // page id of `key` from the LDS table (clamped into it and the cache)
        auto page_entry = [&](int key) __attribute__((always_inline)) {
            const int e = min(max((key >> a.log2_page) - pt_lo, 0), kPrefillBigPages - 1);
            return min(max(sh.pages[e], 0), int32_t(a.num_pages - 1));
        };
        // the wave's 8 rows of tile t (ring position p = t % 3): K and V, four loads
        // byte offset of key `key` of this kv head: a cache row before the
        // split, a new-token row from it on (row key + ext_row0)
        auto key_offset = [&](int key) __attribute__((always_inline)) {
            if (key >= split) return int64_t(key + ext_row0) * slot_bytes + head_bytes;
            const int32_t pg = page_entry(key);
            return int64_t(uint64_t(uint32_t(pg)) * page_bytes) +
                   int32_t((key & page_mask) * slot_bytes + head_bytes);
        };
        auto dma_tile = [&](int t, int p, int32_t pg0) __attribute__((always_inline)) {
            const int key0 = kv_begin + t * BIG_T + 8 * uwave;
            const uint32_t mk = lds_sets + uint32_t(p * BIG_HALF + 8 * uwave * BIG_ROW);
            const uint32_t mv = lds_v + uint32_t(p * BIG_HALF + 8 * uwave * BIG_ROW);
            if (key0 + 7 <= kv_last && key0 + 7 < split && (key0 & page_mask) + 8 <= a.page_size) {
                const int64_t off = int64_t(uint64_t(uint32_t(pg0)) * page_bytes) +
                                    int32_t((key0 & page_mask) * slot_bytes + head_bytes);
                big_dma4(mk, mv, dk0, dk1, dv0, dv1, Kb + off, Vb + off);
            } else if (key0 >= split && key0 + 7 <= kv_last) {
                // eight consecutive new-token rows
                const int64_t off = int64_t(key0 + ext_row0) * slot_bytes + head_bytes;
                big_dma4(mk, mv, dk0, dk1, dv0, dv1, Ke + off, Ve + off);
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int keyk = min(key0 + 4 * i + kr, kv_last);
                    const int keyv = min(key0 + 4 * i + vr, kv_last);
                    const char *bk = keyk >= split ? Ke : Kb;
                    const char *bv = keyv >= split ? Ve : Vb;
                    big_dma1(mk + uint32_t(i * 1024), bk + (key_offset(keyk) + int32_t(i ? kc1 : kc0)));
                    big_dma1(mv + uint32_t(i * 1024), bv + (key_offset(keyv) + int32_t(vc)));
                }
            }
        };
        auto dma_page = [&](int t) __attribute__((always_inline)) {
            return __builtin_amdgcn_readfirstlane(
                page_entry(min(kv_begin + t * BIG_T + 8 * uwave, kv_last)));
        };

        // prologue: page table (of the cached keys), then tiles 0 and 1 landed
        // (step j loads tile j+2)
        {
            const int cache_last = min(kv_last, split - 1);
            const int pt_n = ntiles > 0 && cache_last >= kv_begin
                                 ? min((cache_last >> a.log2_page) - pt_lo + 1, kPrefillBigPages)
                                 : 0;
            for (int e = tid; e < pt_n; e += 512) {
                const int32_t pg = a.kv_indices[page_base + pt_lo + e];
                sh.pages[e] = min(max(pg, 0), int32_t(a.num_pages - 1));
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (ntiles > 0) {
#pragma unroll 1
            for (int t = 0; t < min(ntiles, 2); ++t) dma_tile(t, t, dma_page(t));
            __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();

        // S^T of tile 0, both halves
        f32x16 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[h][i] = 0.f;
        if (ntiles > 0) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    s[h] = mfma32x32x16<F16>(
                        lds_b128((ks & 1 ? kvar1 : kvar0) + uint32_t(h * 32 * BIG_ROW + 256 * (ks >> 1))),
                        qf[ks], s[h]);
        }

        // A 64-key step for tile j is a head and four quarters, in program
        // order fixed by scheduling fences.  S^T(j) is held in two of three
        // 16-register accumulators (half 0 in sb[x], half 1 in sb[y]; sb[z] is
        // free), and the roles rotate (x, y, z) -> (z, x, y) from step to step.
        // The head masks S^T(j) and takes the row maximum.  Quarter q (half
        // h = q/2, 16-key step kk = q%2) runs four MFMAs of S^T(j+1) and then
        // the four P.V MFMAs of its own 16 keys; between the MFMAs the vector
        // ALU makes the four 8-key probability blocks, each block ahead of the
        // P.V MFMAs that use it.
        // S^T(j+1, half 0) goes to sb[z] in quarters 0-1, S^T(j+1, half 1) to
        // sb[x] (free once blocks 0-1 are made) in quarters 2-3.  Quarter 2
        // takes tile j+1's half-0 maximum, so for a tile that needs no mask and
        // no soft cap the head only adds half 1's.
        float mu = 0.f, ahead_max = kNegInf;
        bf16x8 pb[4];
        f32x16 sb[3];
        sb[0] = s[0];
        sb[1] = s[1];
        // two probabilities of block b (scores 8(b%2)+2i, +1 of half b/2)
        auto prob2 = [&](const f32x16 &sh, int b, int i) __attribute__((always_inline)) {
            const int t = 8 * (b & 1) + 2 * i;
            const float p0 = fast_exp2(__builtin_fmaf(sh[t], c, -mu));
            const float p1 = fast_exp2(__builtin_fmaf(sh[t + 1], c, -mu));
            l += p0 + p1;
            // keep the pair's add here, between the MFMAs: left free, the
            // compiler sinks all of a step's adds past its branches into one
            // dependent chain after the last P.V MFMA, where nothing hides it
            asm volatile("" : "+v"(l));
            const bf16x2 pk = to16x2<F16>(f32x2{p0, p1});
            pb[b][2 * i] = pk[0];
            pb[b][2 * i + 1] = pk[1];
        };
        auto head = [&](int j, f32x16 &s0, f32x16 &s1) __attribute__((always_inline)) {
            const int k0 = kv_begin + j * BIG_T;
            const bool interior = k0 + BIG_T <= kv_len &&
                                  (!a.causal || k0 + BIG_T - 1 <= pos0) &&
                                  (W < 0 || k0 >= pos_last - W);
            float mx;
            if (j > 0 && interior && cap_a == 0.f) {
                mx = fmaxf(ahead_max, max16(s1));
            } else {
                if (cap_a != 0.f) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        s0[i] = soft_cap_unit(s0[i], cap_a);
                        s1[i] = soft_cap_unit(s1[i], cap_a);
                    }
                }
                if (!interior) {
                    mask_tile(s0, k0, hw, p_row, kv_len, a.causal, W);
                    mask_tile(s1, k0 + 32, hw, p_row, kv_len, a.causal, W);
                }
                mx = fmaxf(max16(s0), max16(s1));
            }
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                                 __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
            }
            if (__any(mx > m + kRescaleLog2)) {
                const float m_new = fmaxf(m, mx);
                const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m - m_new);
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
                m = m_new;
            }
            mu = m == kNegInf ? 0.f : m;
            __builtin_amdgcn_sched_barrier(0);
        };
        // Operand reads: K operands of S^T(j+1, half h), k-steps kk, kk+2,
        // kk+4, kk+6, and the V^T operands of quarter q of tile j.
        // Each read is issued one MFMA group ahead of its use, into the
        // registers the group before has just consumed: a quarter's K reads
        // follow the previous quarter's QK MFMAs and its V reads follow the
        // previous quarter's P.V MFMAs.  Tile j+1's first K reads wait for the
        // barrier that makes its tile visible; they run under the head.
        bf16x8 kq[4], va[DT];
        // lane bases of the step (copied once per step, so that each read's
        // constant offset stays an immediate of the read)
        uint32_t kv0 = kvar0, kv1 = kvar1, vv = vvar;
        // K operands of S^T(j+1, half h), k-steps kk, kk+2, kk+4, kk+6 (tile
        // j+1 in ring position p1)
        auto load_k = [&](int p1, int q) __attribute__((always_inline)) {
            const int h = q >> 1, kk = q & 1;
            const uint32_t kb = kk ? kv1 : kv0;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                kq[u] = lds_b128(kb + uint32_t(p1 * BIG_HALF + h * 32 * BIG_ROW + 256 * u));
        };
        // V^T operands of quarter q of the tile in ring position p
        auto load_v = [&](int p, int q) __attribute__((always_inline)) {
            const int h = q >> 1, kk = q & 1;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint32_t v0 = vv + uint32_t(p * BIG_HALF + (32 * h + 16 * kk) * BIG_ROW + 256 * dt);
                const i16x4 lo = lds_tr(v0), hi = lds_tr(v0 + 8 * BIG_ROW);
                va[dt] =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        auto quarter = [&](int j, int p, int q, const f32x16 &s0, const f32x16 &s1, f32x16 &dst)
            __attribute__((always_inline)) {
            const int kk = q & 1;
            if (kk == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) dst[i] = 0.f;
            }
            // Block 0 is made during quarter 0's QK MFMAs; block b >= 1 during
            // quarter b-1's P.V MFMAs and quarter b's QK MFMAs (one pair of
            // scores every other MFMA), each ahead of the P.V MFMAs that use it
            // (blocks 0-1: half 0 in s0, blocks 2-3: half 1 in s1), so the
            // vector ALU work is spread over 28 of the step's 32 MFMAs.
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                dst = mfma32x32x16<F16>(kq[u], qf[kk + 2 * u], dst);
                if (q == 0) prob2(s0, 0, u);
                else if (u & 1) prob2(q == 1 ? s0 : s1, q, 2 + (u >> 1));
                __builtin_amdgcn_sched_barrier(0);
            }
            if (q < 3) load_k((p + 1) % 3, q + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                o[u] = mfma32x32x16<F16>(va[u], pb[q], o[u]);
                if (q < 3 && (u & 1)) prob2(q == 0 ? s0 : s1, q + 1, u >> 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (q < 3) load_v(p, q + 1);
            else if (j + 1 < ntiles) load_v((p + 1) % 3, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        // Step j loads tile j+2 into ring position (j+2) % 3, which tile j-1
        // left at the barrier that began the step; it lands before the
        // barrier that ends the step, when tile j+1's K is read next.
        // The page id of the wave's first row of tile j+2 is read from the LDS
        // table one step early (during step j-1), so the loads that begin a
        // step do not wait for an LDS round trip.
        int32_t pg_ahead = page_entry(min(kv_begin + 2 * BIG_T + 8 * uwave, kv_last));
        auto step = [&](int j, int p, f32x16 &sx, f32x16 &sy, f32x16 &sz) __attribute__((always_inline)) {
            if (j + 2 < ntiles) dma_tile(j + 2, (p + 2) % 3, __builtin_amdgcn_readfirstlane(pg_ahead));
            pg_ahead = page_entry(min(kv_begin + (j + 3) * BIG_T + 8 * uwave, kv_last));
            {
                uint32_t x0 = kvar0, x1 = kvar1, x2 = vvar;
                asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2));
                kv0 = x0;
                kv1 = x1;
                vv = x2;
            }
            load_k((p + 1) % 3, 0);
            if (j == 0) load_v(p, 0);
            __builtin_amdgcn_sched_barrier(0);
            head(j, sx, sy);
            quarter(j, p, 0, sx, sy, sz);
            quarter(j, p, 1, sx, sy, sz);
            ahead_max = max16(sz);  // S^T(j+1, half 0) is complete
            quarter(j, p, 2, sx, sy, sx);
            quarter(j, p, 3, sx, sy, sx);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        for (int j = 0; j < ntiles; j += 3) {
            step(j, 0, sb[0], sb[1], sb[2]);
            if (j + 1 < ntiles) step(j + 1, 1, sb[2], sb[0], sb[1]);
            if (j + 2 < ntiles) step(j + 2, 2, sb[1], sb[2], sb[0]);
        }

        l += __shfl_xor(l, 32);
        const int slot0 = w[kPiSlot];
        if (row_valid && slot0 >= 0) {
            // one key chunk of a split tile: the row's partial to its slot
            store_partial<F16>(a, int64_t(slot0 + row_tok * w[kPiSlotStride]) * G + row_head, o,
                               m, l, hw);
        } else if (row_valid) {
            const int64_t lrow = int64_t(q_begin + row_tok) * a.num_qo_heads + hk * G + row_head;
            float w_self = l > 0.f ? a.v_scale / l : 0.f, w_other = 0.f;
            float lse_row = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
            if (a.fold_lse) {
                const Fold f = fold_weights(lse_row, a.fold_lse[lrow]);
                w_self *= f.self;
                w_other = f.other;
                lse_row = f.lse;
            }
            uint16_t *O = static_cast<uint16_t *>(a.o);
            const uint16_t *FO = static_cast<const uint16_t *>(a.fold_o);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int m0 = 0; m0 < 4; ++m0) {
                    const int64_t at = qrow + dt * 32 + 8 * m0 + 4 * hw;
                    f32x4 v4;
#pragma unroll
                    for (int m1 = 0; m1 < 4; ++m1) v4[m1] = o[dt][4 * m0 + m1] * w_self;
                    if (FO) {
                        const f32x4 f4 = from16x4<F16>(*reinterpret_cast<const bf16x4 *>(FO + at));
#pragma unroll
                        for (int m1 = 0; m1 < 4; ++m1) v4[m1] += f4[m1] * w_other;
                    }
                    *reinterpret_cast<bf16x4 *>(O + at) = to16x4<F16>(v4);
                }
            if (a.lse && hw == 0) a.lse[lrow] = lse_row;
        }
        // the loads of the tiles past the last are still in flight: drain them
        // before the next item's prologue rewrites the table and the sets
        if (tid == 0) sh.next_item = claiming ? xcd + kXcds * (xcd_groups + claimed) : n_items;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        it = sh.next_item;
    }
}

// Two workgroups per CU (variant 6: head_dim 128, 4 waves x 32 rows, 16-bit
// K/V, 64-key steps).  The step of prefill_big_kernel (a head, then four
// quarters of S^T(j+1) and P.V MFMAs with the probabilities made between
// them), but with 128 rows per workgroup and two workgroups resident on
// each CU: the two waves that share a SIMD belong to different workgroups,
// whose barriers are independent, so one can run its MFMAs while the other
// runs its softmax or waits at its barrier.  To fit two workgroups in LDS, K
// and V sit in rings of two tiles each (64 KiB): step j loads K(j+2) into the
// slot K(j) left (S^T(j) was made in step j-1) and V(j+1) into the slot
// V(j-1) left, and waits for both at its end.  The page table holds as many
// entries as the plan's longest item can span (dynamic LDS).
constexpr size_t kDuoRingBytes = 4 * size_t(BIG_HALF);  // K ring + V ring

// Four 16-byte row-group loads from one scalar base: blocks m, m + 1 KiB,
// m + 2 KiB, m + 3 KiB (lane offsets d0..d3).  M0 is restored afterwards.
__device__ __forceinline__ void duo_dma4(uint32_t m, uint32_t d0, uint32_t d1, uint32_t d2,
                                         uint32_t d3, const void *base)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %5, %9\n\t"
                 "s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %6, %9\n\t"
                 "s_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %7, %9\n\t"
                 "s_mov_b32 m0, %4\n\tglobal_load_lds_dwordx4 %8, %9\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(m), "s"(m + 1024u), "s"(m + 2048u), "s"(m + 3072u), "v"(d0), "v"(d1),
                   "v"(d2), "v"(d3), "s"(base)
                 : "memory");
}

template <bool F16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_duo_kernel(PrefillArgs a)
{
    constexpr int D = 128, KS = D / 16, DT = D / 32;
    extern __shared__ __attribute__((aligned(1024))) uint8_t duo_lds[];
    int32_t *const pages = reinterpret_cast<int32_t *>(duo_lds + kDuoRingBytes);
    int32_t *const next_item_slot = pages + a.table_pages;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hw = lane >> 5;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int G = 1 << a.log2_group;
    const int n_items = a.ws[kHdrNumItems];
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    const int W = a.window_left;
    const float c = a.scale_log2;
    const float cap_a = a.cap_a;

    const uint32_t lds_k =
        uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void *)duo_lds));
    const uint32_t lds_v = lds_k + uint32_t(2 * BIG_HALF);
    // operand addresses: the chunk-permuted layout of prefill_big_kernel
    const uint32_t kvar0 = lds_k + uint32_t(1024 * (l32 >> 2) + 16 * (l32 & 3) +
                                            64 * ((hw + (l32 >> 2)) & 3));
    const uint32_t kvar1 = lds_k + uint32_t(1024 * (l32 >> 2) + 16 * (l32 & 3) +
                                            64 * ((2 + hw + (l32 >> 2)) & 3));
    const uint32_t vvar = [&] {
        const int e = (lane & 15) >> 2, q = lane & 3, s16 = (lane >> 4) & 1;
        return lds_v + uint32_t(1024 * hw + 64 * e + 16 * (2 * s16 + (q >> 1)) + 8 * (q & 1));
    }();
    // staging: wave w stages keys 16w .. 16w+15 of a tile, four 1 KiB blocks
    // b = 4w + i of four rows; lane L writes LDS byte 16L of the block and
    // fetches K: row L % 4, chunk 4 (L / 16) + ((L / 4 - i) % 4);
    //         V: row (L / 4) % 4, chunk 4 (L / 16) + L % 4
    const int64_t slot_stride = int64_t(a.num_kv_heads) * D;
    const int32_t slot_bytes = int32_t(slot_stride * 2);
    const uint32_t page_bytes = uint32_t(slot_stride * a.page_rows * 2);
    const int kr = lane & 3, vr = (lane >> 2) & 3;
    uint32_t kc[4], dk[4], dv[4];
    const uint32_t vc = uint32_t(16 * (4 * (lane >> 4) + (lane & 3)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kc[i] = uint32_t(16 * (4 * (lane >> 4) + (((lane >> 2) - i) & 3)));
        dk[i] = uint32_t((4 * i + kr) * slot_bytes) + kc[i];
        dv[i] = uint32_t((4 * i + vr) * slot_bytes) + vc;
    }
    const char *const Kb = static_cast<const char *>(a.k);
    const char *const Vb = static_cast<const char *>(a.v);
    const int page_mask = a.page_size - 1;
    const int table_last = a.table_pages - 1;

    // run-time item claiming per XCD, as prefill_big_kernel
    int32_t *const ctr = a.ws;
    const int xcd = blockIdx.x % kXcds;
    const int xcd_groups = (int(gridDim.x) - xcd + kXcds - 1) / kXcds;
    if (int(blockIdx.x) >= n_items) return;
    // With a workgroup for every item nothing is handed out and the counters
    // are not touched.  Otherwise each processed item starts with one claim
    // on its XCD's counter, so that counter sees exactly as many claims as
    // the XCD has items, returning 0 .. n-1: the workgroup that draws n-1
    // makes its last claim and puts it back to 0 for the next launch.
    const bool claiming = int(gridDim.x) < n_items;
    const int xcd_items = (n_items - xcd + kXcds - 1) / kXcds;
    for (int it = blockIdx.x; it < n_items;) {
        int claimed = 0;
        if (claiming && tid == 0) {
            claimed = atomicAdd(ctr + kHdrNextItem + xcd, 1);
            if (claimed == xcd_items - 1) ctr[kHdrNextItem + xcd] = 0;
        }
        const int32_t *w = a.ws + kHeaderWords + int64_t(it) * kPrefillItemWords;
        const int hk = w[kPiKvHead], q_begin = w[kPiQBegin], q_count = w[kPiQCount];
        const int pos0 = w[kPiPos0], kv_len = w[kPiKvLen];
        const int kv_begin = w[kPiKvBegin];
        const int page_base = w[kPiPageBase];
        const int kv_end = a.causal ? min(kv_len, pos0 + q_count) : kv_len;
        const int pos_last = pos0 + q_count - 1;
        const int ntiles = kv_end > kv_begin ? (kv_end - kv_begin + BIG_T - 1) / BIG_T : 0;
        const int pt_lo = kv_begin >> a.log2_page;
        const int32_t head_bytes = int32_t(hk * D * 2);
        const int kv_last = min(kv_begin + ntiles * BIG_T, kv_len) - 1;

        const int row = wave * 32 + l32;
        const int row_tok = row >> a.log2_group, row_head = row & (G - 1);
        const bool row_valid = row_tok < q_count;
        const int p_row = pos0 + row_tok;
        const int64_t qrow = (int64_t(q_begin + row_tok) * a.num_qo_heads + hk * G + row_head) * D;
        bf16x8 qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = row_valid ? load_bf16x8(Q + qrow + ks * 16 + hw * 8) : zero_bf16x8();

        float m = kNegInf, l = 0.f;
        f32x16 o[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

        auto page_entry = [&](int key) __attribute__((always_inline)) {
            const int e = min(max((key >> a.log2_page) - pt_lo, 0), table_last);
            return min(max(pages[e], 0), int32_t(a.num_pages - 1));
        };
        // the wave's 16 rows of tile t of one tensor (K: base Kb, V: Vb) into
        // the LDS tile at `set`
        auto dma_rows = [&](int t, uint32_t set, const char *base, const uint32_t (&d)[4],
                            bool is_k) __attribute__((always_inline)) {
            const int key0 = kv_begin + t * BIG_T + 16 * uwave;
            const uint32_t mrow = set + uint32_t(16 * uwave * BIG_ROW);
            const int32_t pg0 = __builtin_amdgcn_readfirstlane(page_entry(min(key0, kv_last)));
            if (key0 + 15 <= kv_last && (key0 & page_mask) + 16 <= a.page_size) {
                const int64_t off = int64_t(uint64_t(uint32_t(pg0)) * page_bytes) +
                                    int32_t((key0 & page_mask) * slot_bytes + head_bytes);
                duo_dma4(mrow, d[0], d[1], d[2], d[3], base + off);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = min(key0 + 4 * i + (is_k ? kr : vr), kv_last);
                    const int32_t pg = page_entry(key);
                    const int64_t off = int64_t(uint64_t(uint32_t(pg)) * page_bytes) +
                                        int32_t((key & page_mask) * slot_bytes + head_bytes);
                    big_dma1(mrow + uint32_t(i * 1024),
                             base + (off + int32_t(is_k ? kc[i] : vc)));
                }
            }
        };
        auto dma_k = [&](int t, int p) __attribute__((always_inline)) {
            dma_rows(t, lds_k + uint32_t(p * BIG_HALF), Kb, dk, true);
        };
        auto dma_v = [&](int t, int p) __attribute__((always_inline)) {
            dma_rows(t, lds_v + uint32_t(p * BIG_HALF), Vb, dv, false);
        };

        // prologue: page table, then K(0), K(1) and V(0) landed
        {
            const int pt_n =
                ntiles > 0 ? min((kv_last >> a.log2_page) - pt_lo + 1, a.table_pages) : 0;
            for (int e = tid; e < pt_n; e += 256) {
                const int32_t pg = a.kv_indices[page_base + pt_lo + e];
                pages[e] = min(max(pg, 0), int32_t(a.num_pages - 1));
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (ntiles > 0) {
            dma_k(0, 0);
            if (ntiles > 1) dma_k(1, 1);
            dma_v(0, 0);
            __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();

        // S^T of tile 0, both halves
        f32x16 s[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[h][i] = 0.f;
        if (ntiles > 0) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    s[h] = mfma32x32x16<F16>(
                        lds_b128((ks & 1 ? kvar1 : kvar0) + uint32_t(h * 32 * BIG_ROW + 256 * (ks >> 1))),
                        qf[ks], s[h]);
        }
        // step 0 loads K(2) into K(0)'s slot: every wave's reads of K(0) first
        __syncthreads();

        float mu = 0.f, ahead_max = kNegInf;
        bf16x8 pb[4];
        f32x16 sb[3];
        sb[0] = s[0];
        sb[1] = s[1];
        auto prob2 = [&](const f32x16 &sh, int b, int i) __attribute__((always_inline)) {
            const int t = 8 * (b & 1) + 2 * i;
            const float p0 = fast_exp2(__builtin_fmaf(sh[t], c, -mu));
            const float p1 = fast_exp2(__builtin_fmaf(sh[t + 1], c, -mu));
            l += p0 + p1;
            const bf16x2 pk = to16x2<F16>(f32x2{p0, p1});
            pb[b][2 * i] = pk[0];
            pb[b][2 * i + 1] = pk[1];
        };
        auto head = [&](int j, f32x16 &s0, f32x16 &s1) __attribute__((always_inline)) {
            const int k0 = kv_begin + j * BIG_T;
            const bool interior = k0 + BIG_T <= kv_len &&
                                  (!a.causal || k0 + BIG_T - 1 <= pos0) &&
                                  (W < 0 || k0 >= pos_last - W);
            float mx;
            if (j > 0 && interior && cap_a == 0.f) {
                mx = fmaxf(ahead_max, max16(s1));
            } else {
                if (cap_a != 0.f) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        s0[i] = soft_cap_unit(s0[i], cap_a);
                        s1[i] = soft_cap_unit(s1[i], cap_a);
                    }
                }
                if (!interior) {
                    mask_tile(s0, k0, hw, p_row, kv_len, a.causal, W);
                    mask_tile(s1, k0 + 32, hw, p_row, kv_len, a.causal, W);
                }
                mx = fmaxf(max16(s0), max16(s1));
            }
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                                 __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
            }
            if (__any(mx > m + kRescaleLog2)) {
                const float m_new = fmaxf(m, mx);
                const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m - m_new);
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
                m = m_new;
            }
            mu = m == kNegInf ? 0.f : m;
            __builtin_amdgcn_sched_barrier(0);
        };
        bf16x8 kq[4], va[DT];
        uint32_t kv0 = kvar0, kv1 = kvar1, vv = vvar;
        // K operands of S^T(j+1, half h), k-steps kk, kk+2, kk+4, kk+6 (K slot pk)
        auto load_k = [&](int pk, int q) __attribute__((always_inline)) {
            const int h = q >> 1, kk = q & 1;
            const uint32_t kb = kk ? kv1 : kv0;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                kq[u] = lds_b128(kb + uint32_t(pk * BIG_HALF + h * 32 * BIG_ROW + 256 * u));
        };
        // V^T operands of quarter q of the tile in V slot pv
        auto load_v = [&](int pv, int q) __attribute__((always_inline)) {
            const int h = q >> 1, kk = q & 1;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint32_t v0 = vv + uint32_t(pv * BIG_HALF + (32 * h + 16 * kk) * BIG_ROW + 256 * dt);
                const i16x4 lo = lds_tr(v0), hi = lds_tr(v0 + 8 * BIG_ROW);
                va[dt] =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        auto quarter = [&](int pk, int pv, int q, const f32x16 &s0, const f32x16 &s1, f32x16 &dst)
            __attribute__((always_inline)) {
            const int kk = q & 1;
            if (kk == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) dst[i] = 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                dst = mfma32x32x16<F16>(kq[u], qf[kk + 2 * u], dst);
                if (q < 2) prob2(q == 0 ? s0 : s1, 2 * q, u);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (q < 3) load_k(pk, q + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                o[u] = mfma32x32x16<F16>(va[u], pb[q], o[u]);
                if (q < 2) prob2(q == 0 ? s0 : s1, 2 * q + 1, u);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (q < 3) load_v(pv, q + 1);
            __builtin_amdgcn_sched_barrier(0);
        };
        // Step j: K(j+1) in slot pk = (j+1) % 2, V(j) in slot pv = j % 2.  It
        // loads K(j+2) into slot pv (K(j) is no longer read) and V(j+1) into
        // slot pk (V(j-1) is no longer read), and waits for them at its end.
        auto step = [&](int j, int pk, int pv, f32x16 &sx, f32x16 &sy, f32x16 &sz)
            __attribute__((always_inline)) {
            if (j + 2 < ntiles) dma_k(j + 2, pv);
            if (j + 1 < ntiles) dma_v(j + 1, pk);
            {
                uint32_t x0 = kvar0, x1 = kvar1, x2 = vvar;
                asm volatile("" : "+v"(x0), "+v"(x1), "+v"(x2));
                kv0 = x0;
                kv1 = x1;
                vv = x2;
            }
            load_k(pk, 0);
            load_v(pv, 0);
            __builtin_amdgcn_sched_barrier(0);
            head(j, sx, sy);
            quarter(pk, pv, 0, sx, sy, sz);
            quarter(pk, pv, 1, sx, sy, sz);
            ahead_max = max16(sz);  // S^T(j+1, half 0) is complete
            quarter(pk, pv, 2, sx, sy, sx);
            quarter(pk, pv, 3, sx, sy, sx);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        // unrolled by six: the slots repeat every two steps, the score
        // accumulators' roles every three
        for (int j = 0; j < ntiles; j += 6) {
            step(j, 1, 0, sb[0], sb[1], sb[2]);
            if (j + 1 < ntiles) step(j + 1, 0, 1, sb[2], sb[0], sb[1]);
            if (j + 2 < ntiles) step(j + 2, 1, 0, sb[1], sb[2], sb[0]);
            if (j + 3 < ntiles) step(j + 3, 0, 1, sb[0], sb[1], sb[2]);
            if (j + 4 < ntiles) step(j + 4, 1, 0, sb[2], sb[0], sb[1]);
            if (j + 5 < ntiles) step(j + 5, 0, 1, sb[1], sb[2], sb[0]);
        }

        l += __shfl_xor(l, 32);
        if (row_valid) {
            const int64_t lrow = int64_t(q_begin + row_tok) * a.num_qo_heads + hk * G + row_head;
            float w_self = l > 0.f ? a.v_scale / l : 0.f, w_other = 0.f;
            float lse_row = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
            if (a.fold_lse) {
                const Fold f = fold_weights(lse_row, a.fold_lse[lrow]);
                w_self *= f.self;
                w_other = f.other;
                lse_row = f.lse;
            }
            uint16_t *O = static_cast<uint16_t *>(a.o);
            const uint16_t *FO = static_cast<const uint16_t *>(a.fold_o);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int m0 = 0; m0 < 4; ++m0) {
                    const int64_t at = qrow + dt * 32 + 8 * m0 + 4 * hw;
                    f32x4 v4;
#pragma unroll
                    for (int m1 = 0; m1 < 4; ++m1) v4[m1] = o[dt][4 * m0 + m1] * w_self;
                    if (FO) {
                        const f32x4 f4 = from16x4<F16>(*reinterpret_cast<const bf16x4 *>(FO + at));
#pragma unroll
                        for (int m1 = 0; m1 < 4; ++m1) v4[m1] += f4[m1] * w_other;
                    }
                    *reinterpret_cast<bf16x4 *>(O + at) = to16x4<F16>(v4);
                }
            if (a.lse && hw == 0) a.lse[lrow] = lse_row;
        }
        if (tid == 0) *next_item_slot = claiming ? xcd + kXcds * (xcd_groups + claimed) : n_items;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        it = *next_item_slot;
    }
}

// fp32 inputs: one wave per (query token, head) row, keys visited in order
// with a running maximum, all arithmetic in fp32.
__global__ __launch_bounds__(kGenericThreads) void attention_fp32_kernel(PrefillArgs a, int D)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int G = 1 << a.log2_group;
    const int n_items = a.ws[kHdrNumItems];
    const float *Q = static_cast<const float *>(a.q);
    const float *K = static_cast<const float *>(a.k);
    const float *V = static_cast<const float *>(a.v);
    float *O = static_cast<float *>(a.o);
    const int W = a.window_left, P = a.page_size;
    const int E = D / 64;  // dims per lane (1, 2 or 4)

    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const int32_t *w = a.ws + kHeaderWords + int64_t(it) * kPrefillItemWords;
        const int hk = w[kPiKvHead], q_begin = w[kPiQBegin], q_count = w[kPiQCount];
        const int pos0 = w[kPiPos0], kv_len = w[kPiKvLen], page_base = w[kPiPageBase];
        for (int row = wave; row < q_count * G; row += kGenericThreads / 64) {
            const int tok = row / G, h = hk * G + row % G;
            const int p = pos0 + tok;
            const int64_t qrow = (int64_t(q_begin + tok) * a.num_qo_heads + h) * D;
            float q[4], acc[4];
            for (int e = 0; e < 4; ++e) {
                q[e] = e < E ? Q[qrow + lane + 64 * e] : 0.f;
                acc[e] = 0.f;
            }
            int lo = W >= 0 ? max(0, p - W) : 0;
            int hi = a.causal ? min(p, kv_len - 1) : kv_len - 1;
            float m = kNegInf, l = 0.f;
            for (int j = lo; j <= hi; ++j) {
                const int64_t pg = page_of(a.kv_indices, page_base, j, a.log2_page, a.num_pages);
                const int64_t off = nhd_offset(pg, j & (P - 1), a.page_rows, hk, a.num_kv_heads, D);
                float dot = 0.f;
                for (int e = 0; e < E; ++e) dot += q[e] * K[off + lane + 64 * e];
                for (int s = 32; s >= 1; s >>= 1) dot += __shfl_xor(dot, s);
                const float x = (a.cap_a != 0.f ? soft_cap_unit(dot, a.cap_a) : dot) * a.scale_log2;
                const float m_new = fmaxf(m, x);
                const float alpha = fast_exp2(m - m_new);
                const float pj = fast_exp2(x - m_new);
                l = l * alpha + pj;
                for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + pj * V[off + lane + 64 * e];
                m = m_new;
            }
            const int64_t lrow = int64_t(q_begin + tok) * a.num_qo_heads + h;
            float w_self = l > 0.f ? a.v_scale / l : 0.f, w_other = 0.f;
            float lse_row = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
            if (a.fold_lse) {
                const Fold f = fold_weights(lse_row, a.fold_lse[lrow]);
                w_self *= f.self;
                w_other = f.other;
                lse_row = f.lse;
            }
            const float *FO = static_cast<const float *>(a.fold_o);
            for (int e = 0; e < E; ++e) {
                const int64_t at = qrow + lane + 64 * e;
                O[at] = acc[e] * w_self + (FO ? FO[at] * w_other : 0.f);
            }
            if (a.lse && lane == 0) a.lse[lrow] = lse_row;
        }
    }
}

}  // namespace

size_t prefill_duo_lds_bytes(int table_pages)
{
    return kDuoRingBytes + 4 * size_t(table_pages) + 16;
}

template <bool F16, int KVF>
static hipError_t launch_prefill_t(const PrefillArgs &a, int head_dim, int variant, int grid,
                                   hipStream_t s)
{
    if constexpr (KVF == 0) {
        if (variant == kPrefillDma) {
            if (head_dim != 128) return hipErrorInvalidValue;
            prefill_kernel<128, 8, true, F16, 0><<<grid, 512, 0, s>>>(a);
            return hipGetLastError();
        }
        if (variant == kPrefillBig) {
            if (head_dim != 128) return hipErrorInvalidValue;
            prefill_big_kernel<F16><<<grid, 512, 0, s>>>(a);
            return hipGetLastError();
        }
        if (variant == kPrefillDuo) {
            if (head_dim != 128 || a.table_pages < 1 || a.table_pages > kPrefillDmaPages)
                return hipErrorInvalidValue;
            prefill_duo_kernel<F16><<<grid, 256, prefill_duo_lds_bytes(a.table_pages), s>>>(a);
            return hipGetLastError();
        }

        if (variant == kPrefillWide) {
            switch (head_dim) {
            case 64: prefill_wide_kernel<64, F16><<<grid, 256, 0, s>>>(a); break;
            case 128: prefill_wide_kernel<128, F16><<<grid, 256, 0, s>>>(a); break;
            default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
    } else if (variant == kPrefillDma || variant == kPrefillWide || variant == kPrefillBig ||
               variant == kPrefillDuo) {
        return hipErrorInvalidValue;  // 8-bit K/V are widened on the register-staged path
    }
    if (variant == kPrefillRows256) {
        switch (head_dim) {
        case 64: prefill_kernel<64, 8, false, F16, KVF><<<grid, 512, 0, s>>>(a); break;
        case 128: prefill_kernel<128, 8, false, F16, KVF><<<grid, 512, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (head_dim) {
        case 64: prefill_kernel<64, 4, false, F16, KVF><<<grid, 256, 0, s>>>(a); break;
        case 128: prefill_kernel<128, 4, false, F16, KVF><<<grid, 256, 0, s>>>(a); break;
        case 256: prefill_kernel<256, 4, false, F16, KVF><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <bool F16>
static hipError_t launch_prefill_f(const PrefillArgs &a, int head_dim, int variant, int kv_format,
                                   int grid, hipStream_t s)
{
    switch (kv_format) {
    case 0: return launch_prefill_t<F16, 0>(a, head_dim, variant, grid, s);
    case PKVS_KV_FP8_E4M3: return launch_prefill_t<F16, 1>(a, head_dim, variant, grid, s);
    case PKVS_KV_FP8_E5M2: return launch_prefill_t<F16, 2>(a, head_dim, variant, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_16bit(const PrefillArgs &a, int head_dim, int variant, bool f16,
                                int kv_format, int grid, hipStream_t s)
{
    return f16 ? launch_prefill_f<true>(a, head_dim, variant, kv_format, grid, s)
               : launch_prefill_f<false>(a, head_dim, variant, kv_format, grid, s);
}

hipError_t launch_attention_fp32(const PrefillArgs &a, int head_dim, int grid, hipStream_t s)
{
    attention_fp32_kernel<<<grid, kGenericThreads, 0, s>>>(a, head_dim);
    return hipGetLastError();
}

template <typename K>
static int blocks_per_cu(K kernel, int threads)
{
    int n = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) == hipSuccess ? n
                                                                                             : 0;
}

template <bool F16, int KVF>
static int prefill_blocks_per_cu_t(int head_dim, int variant, int table_pages)
{
    if constexpr (KVF == 0) {
        if (variant == kPrefillDma)
            return head_dim == 128 ? blocks_per_cu(prefill_kernel<128, 8, true, F16, 0>, 512) : 0;
        if (variant == kPrefillBig)
            return head_dim == 128 ? blocks_per_cu(prefill_big_kernel<F16>, 512) : 0;
        if (variant == kPrefillDuo) {
            int n = 0;
            return head_dim == 128 &&
                           hipOccupancyMaxActiveBlocksPerMultiprocessor(
                               &n, prefill_duo_kernel<F16>, 256,
                               prefill_duo_lds_bytes(table_pages)) == hipSuccess
                       ? n
                       : 0;
        }

        if (variant == kPrefillWide) {
            if (head_dim == 64) return blocks_per_cu(prefill_wide_kernel<64, F16>, 256);
            if (head_dim == 128) return blocks_per_cu(prefill_wide_kernel<128, F16>, 256);
            return 0;
        }
    } else if (variant == kPrefillDma || variant == kPrefillWide || variant == kPrefillBig ||
               variant == kPrefillDuo) {
        return 0;
    }
    if (variant == kPrefillRows256) {
        if (head_dim == 64) return blocks_per_cu(prefill_kernel<64, 8, false, F16, KVF>, 512);
        if (head_dim == 128) return blocks_per_cu(prefill_kernel<128, 8, false, F16, KVF>, 512);
        return 0;
    }
    if (head_dim == 64) return blocks_per_cu(prefill_kernel<64, 4, false, F16, KVF>, 256);
    if (head_dim == 128) return blocks_per_cu(prefill_kernel<128, 4, false, F16, KVF>, 256);
    if (head_dim == 256) return blocks_per_cu(prefill_kernel<256, 4, false, F16, KVF>, 256);
    return 0;
}

template <bool F16>
static int prefill_blocks_per_cu_f(int head_dim, int variant, int kv_format, int table_pages)
{
    switch (kv_format) {
    case 0: return prefill_blocks_per_cu_t<F16, 0>(head_dim, variant, table_pages);
    case PKVS_KV_FP8_E4M3: return prefill_blocks_per_cu_t<F16, 1>(head_dim, variant, table_pages);
    case PKVS_KV_FP8_E5M2: return prefill_blocks_per_cu_t<F16, 2>(head_dim, variant, table_pages);
    default: return 0;
    }
}

int prefill_blocks_per_cu(int head_dim, int variant, bool f16, int kv_format, int table_pages)
{
    return f16 ? prefill_blocks_per_cu_f<true>(head_dim, variant, kv_format, table_pages)
               : prefill_blocks_per_cu_f<false>(head_dim, variant, kv_format, table_pages);
}

}  // namespace pkvs
