// prefill.hip -- causal paged prefill (extend with a cached prefix) with the
// exact sliding-window mask, for gfx950.
//
// bf16 path: one workgroup (4 waves) owns one work item = (request, kv head,
// tile of 128/G query tokens).  The G query heads of the kv head are packed
// with the tokens into 128 rows (row = token * G + head), so a K/V tile staged
// in LDS serves all of them.  Each wave owns 32 rows and runs
//     S^T[32 keys x 32 rows] = K[32 keys x D] . Q^T[D x 32 rows]
//     O^T[32 dims x 32 rows] += V^T[32 dims x 32 keys] . P^T[32 keys x 32 rows]
// on v_mfma_f32_32x32x16_bf16.  With S^T (keys in M) every lane holds 16 keys
// of one row, so the row maximum and sum are lane-local plus one exchange
// with the lane 32 away, and the probabilities are already laid out as the B
// operand of the PV product.  K sits in LDS row-major (A operand reads 16
// bytes of one key), V is transposed while it is staged (A operand reads
// 8 bytes = 4 keys of one dim).
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
// fp32 path (attention_fp32_kernel): a plain wave-per-row loop in fp32 for
// fp32 inputs, used for small correctness-critical problems; it serves both
// prefill items and decode (as one-query items).
#include "device_common.h"
#include "pkvs_internal.h"

namespace pkvs {

namespace {

constexpr int KT = kPrefillKvTile;
constexpr int KPAD = 8;  // bf16 of padding per K row in LDS
constexpr int VPAD = 4;  // bf16 of padding per V^T row in LDS (rows of 36 = 18 dwords)

template <int D>
struct PrefillLds {
    uint16_t k[KT][D + KPAD];
    uint16_t vt[D][KT + VPAD];
};

template <int D>
struct TileRegs {
    static constexpr int KCH = KT * D / 8 / kPrefillThreads;   // 16-byte K chunks per thread
    static constexpr int VBLK = (D + kPrefillThreads - 1) / kPrefillThreads;  // 4x8 V blocks
    u32x4 k[KCH > 0 ? KCH : 1];
    u32x4 v[VBLK][4];
};

// Page ids of the keys this thread stages for one tile (K chunks and one V
// block), fetched a tile ahead of the K/V loads that use them so the
// dependent index load never sits on the critical path.
template <int D>
struct TilePages {
    int64_t k[TileRegs<D>::KCH > 0 ? TileRegs<D>::KCH : 1];
    int64_t v[4];
};

template <int D>
__device__ __forceinline__ void pages_load(TilePages<D> &pg, const PrefillArgs &a, int k0,
                                           int kv_len, int page_base, int tid)
{
    constexpr int KCH = TileRegs<D>::KCH;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        const int key = min(k0 + (tid + i * kPrefillThreads) / CPR, kv_len - 1);
        pg.k[i] = page_of(a.kv_indices, page_base, max(key, 0), a.log2_page, a.num_pages);
    }
    const int kq = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = min(k0 + 4 * kq + i, kv_len - 1);
        pg.v[i] = (a.page_size >= 4 && i > 0)
                      ? pg.v[0]
                      : page_of(a.kv_indices, page_base, max(key, 0), a.log2_page, a.num_pages);
    }
}

// Global -> registers for the key tile starting at k0, at the pages in pg.
// Keys outside [0, kv_len) are zero-filled so that no unwritten slot (which
// may hold any bits, even NaN) ever reaches the MFMA.
template <int D>
__device__ __forceinline__ void tile_load(TileRegs<D> &t, const TilePages<D> &pg,
                                          const PrefillArgs &a, int k0, int kv_len, int hk,
                                          int tid)
{
    constexpr int KCH = TileRegs<D>::KCH, VBLK = TileRegs<D>::VBLK;
    constexpr int CPR = D / 8;  // 16-byte chunks per key row
    const uint16_t *K = static_cast<const uint16_t *>(a.k);
    const uint16_t *V = static_cast<const uint16_t *>(a.v);
    const int P = a.page_size;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        const int c = tid + i * kPrefillThreads;
        const int key = k0 + c / CPR, ch = c % CPR;
        t.k[i] = key < kv_len
                     ? *reinterpret_cast<const u32x4 *>(
                           K + nhd_offset(pg.k[i], key & (P - 1), P, hk, a.num_kv_heads, D) +
                           ch * 8)
                     : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int bi = 0; bi < VBLK; ++bi) {
        const int c = tid + bi * kPrefillThreads;  // block: 4 keys x 8 dims
        if (c < D) {
            const int kq = c & 7, ch = c >> 3;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = k0 + 4 * kq + i;
                t.v[bi][i] = key < kv_len
                                 ? *reinterpret_cast<const u32x4 *>(
                                       V + nhd_offset(pg.v[i], key & (P - 1), P, hk,
                                                      a.num_kv_heads, D) +
                                       ch * 8)
                                 : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
}

// Registers -> LDS; V is transposed on the way (4 keys x 8 dims -> 8 rows of
// 4 keys).
template <int D>
__device__ __forceinline__ void tile_store(const TileRegs<D> &t, PrefillLds<D> &s, int tid)
{
    constexpr int KCH = TileRegs<D>::KCH, VBLK = TileRegs<D>::VBLK;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        const int c = tid + i * kPrefillThreads;
        *reinterpret_cast<u32x4 *>(&s.k[c / CPR][(c % CPR) * 8]) = t.k[i];
    }
#pragma unroll
    for (int bi = 0; bi < VBLK; ++bi) {
        const int c = tid + bi * kPrefillThreads;
        if (c < D) {
            const int kq = c & 7, ch = c >> 3;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // dim ch*8+e of keys 4kq..4kq+3: 16-bit halves of the rows' dword e/2
                const int sh = (e & 1) * 16;
                const uint32_t x0 = (t.v[bi][0][e >> 1] >> sh) & 0xffffu;
                const uint32_t x1 = (t.v[bi][1][e >> 1] >> sh) & 0xffffu;
                const uint32_t x2 = (t.v[bi][2][e >> 1] >> sh) & 0xffffu;
                const uint32_t x3 = (t.v[bi][3][e >> 1] >> sh) & 0xffffu;
                *reinterpret_cast<u32x2 *>(&s.vt[ch * 8 + e][4 * kq]) =
                    u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_bf16_kernel(PrefillArgs a)
{
    constexpr int KSTEPS = D / 16;  // QK k-steps
    constexpr int DT = D / 32;      // O^T dim tiles
    __shared__ __attribute__((aligned(16))) PrefillLds<D> lds;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hw = lane >> 5;
    const int G = 1 << a.log2_group;
    const int n_items = a.ws[kHdrNumItems];
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    const int W = a.window_left;

    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const int32_t *w = a.ws + kHeaderWords + int64_t(it) * kPrefillItemWords;
        const int hk = w[kPiKvHead], q_begin = w[kPiQBegin], q_count = w[kPiQCount];
        const int pos0 = w[kPiPos0], kv_len = w[kPiKvLen], page_base = w[kPiPageBase];
        const int kv_begin = w[kPiKvBegin];
        const int kv_end = a.causal ? min(kv_len, pos0 + q_count) : kv_len;
        const int pos_last = pos0 + q_count - 1;

        // this lane's row (both S^T and O^T keep one row per lane: column l32)
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

        TileRegs<D> regs;
        TilePages<D> pages;
        if (kv_begin < kv_end) {
            pages_load<D>(pages, a, kv_begin, kv_len, page_base, tid);
            tile_load<D>(regs, pages, a, kv_begin, kv_len, hk, tid);
            pages_load<D>(pages, a, kv_begin + KT, kv_len, page_base, tid);
        }

        for (int k0 = kv_begin; k0 < kv_end; k0 += KT) {
            __syncthreads();  // every wave is done reading the previous tile
            tile_store<D>(regs, lds, tid);
            __syncthreads();
            if (k0 + KT < kv_end) {
                tile_load<D>(regs, pages, a, k0 + KT, kv_len, hk, tid);
                pages_load<D>(pages, a, k0 + 2 * KT, kv_len, page_base, tid);
            }

            // S^T = K . Q^T
            f32x16 sacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&lds.k[l32][ks * 16 + hw * 8]);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc, 0, 0, 0);
            }

            // key of accumulator entry i = 4*m0 + m1: k0 + 8*m0 + 4*hw + m1
            const bool interior = k0 + KT <= kv_len && (!a.causal || k0 + KT - 1 <= pos0) &&
                                  (W < 0 || k0 >= pos_last - W);
            float x[16];
            float mx = kNegInf;
            if (interior) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    x[i] = sacc[i] * a.scale_log2;
                    mx = fmaxf(mx, x[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 8 * (i >> 2) + 4 * hw + (i & 3);
                    const bool vis = key < kv_len && (!a.causal || key <= p_row) &&
                                     (W < 0 || key >= p_row - W);
                    x[i] = vis ? sacc[i] * a.scale_log2 : kNegInf;
                    mx = fmaxf(mx, x[i]);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m, mx);
            const float m_use = m_new == kNegInf ? 0.f : m_new;
            const float alpha = fast_exp2(m - m_use);
            float rs = 0.f;
            f32x16 pr;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                pr[i] = fast_exp2(x[i] - m_use);
                rs += pr[i];
            }
            l = l * alpha + rs;
            m = m_new;

            // O^T += V^T . P^T, two k-steps of 16 keys
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                f32x8 p8;
#pragma unroll
                for (int j = 0; j < 8; ++j) p8[j] = pr[8 * kk + j];
                const bf16x8 pb = __builtin_convertvector(p8, bf16x8);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int d = dt * 32 + l32;
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(&lds.vt[d][16 * kk + 4 * hw]);
                    const u32x2 hi =
                        *reinterpret_cast<const u32x2 *>(&lds.vt[d][16 * kk + 8 + 4 * hw]);
                    const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                    f32x16 c = o[dt];
                    if (kk == 0) c *= alpha;
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, c, 0, 0, 0);
                }
            }
        }

        // epilogue: rows are split over the two half-waves' key sets
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (row_valid) {
            uint16_t *O = static_cast<uint16_t *>(a.o);
            const int64_t orow = qrow;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int m0 = 0; m0 < 4; ++m0) {
                    f32x4 v4;
#pragma unroll
                    for (int m1 = 0; m1 < 4; ++m1) v4[m1] = o[dt][4 * m0 + m1] * inv;
                    *reinterpret_cast<bf16x4 *>(O + orow + dt * 32 + 8 * m0 + 4 * hw) =
                        __builtin_convertvector(v4, bf16x4);
                }
            if (a.lse && hw == 0)
                a.lse[int64_t(q_begin + row_tok) * a.num_qo_heads + hk * G + row_head] =
                    l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
        }
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
                const int64_t off = nhd_offset(pg, j & (P - 1), P, hk, a.num_kv_heads, D);
                float dot = 0.f;
                for (int e = 0; e < E; ++e) dot += q[e] * K[off + lane + 64 * e];
                for (int s = 32; s >= 1; s >>= 1) dot += __shfl_xor(dot, s);
                const float x = dot * a.scale_log2;
                const float m_new = fmaxf(m, x);
                const float alpha = fast_exp2(m - m_new);
                const float pj = fast_exp2(x - m_new);
                l = l * alpha + pj;
                for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + pj * V[off + lane + 64 * e];
                m = m_new;
            }
            const float inv = l > 0.f ? 1.f / l : 0.f;
            for (int e = 0; e < E; ++e) O[qrow + lane + 64 * e] = acc[e] * inv;
            if (a.lse && lane == 0)
                a.lse[int64_t(q_begin + tok) * a.num_qo_heads + h] =
                    l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, int grid, hipStream_t s)
{
    switch (head_dim) {
    case 64: prefill_bf16_kernel<64><<<grid, kPrefillThreads, 0, s>>>(a); break;
    case 128: prefill_bf16_kernel<128><<<grid, kPrefillThreads, 0, s>>>(a); break;
    case 256: prefill_bf16_kernel<256><<<grid, kPrefillThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attention_fp32(const PrefillArgs &a, int head_dim, int grid, hipStream_t s)
{
    attention_fp32_kernel<<<grid, kGenericThreads, 0, s>>>(a, head_dim);
    return hipGetLastError();
}

int prefill_bf16_blocks_per_cu(int head_dim)
{
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (head_dim) {
    case 64:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<64>,
                                                         kPrefillThreads, 0);
        break;
    case 128:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<128>,
                                                         kPrefillThreads, 0);
        break;
    case 256:
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<256>,
                                                         kPrefillThreads, 0);
        break;
    }
    return e == hipSuccess ? n : 0;
}

}  // namespace pkvs
