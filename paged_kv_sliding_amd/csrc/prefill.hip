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
// Three key tiles are in flight in LDS (one barrier per tile): while tile j's
// softmax runs, the MFMAs of tile j+1's S^T are already issued, tile j+2 is
// being written to LDS and tile j+3 read from HBM into registers.
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
// fp32 path (attention_fp32_kernel): a plain wave-per-row loop in fp32 for
// fp32 inputs, used for small correctness-critical problems; it serves both
// prefill items and decode (as one-query items).
#include "device_common.h"
#include "pkvs_internal.h"

namespace pkvs {

namespace {

constexpr int KT = kPrefillKvTile;
constexpr int KPAD = 8;                // K rows: D+8 bf16, a stride of 4 dwords mod 64 banks
constexpr int VPAD = 32;               // V rows: D+32 bf16, a stride of 16 dwords mod 64 banks
constexpr int NBUF = 3;                // LDS tile sets in flight
constexpr float kRescaleLog2 = 8.0f;   // rescale O only when a row max grows by > 2^8

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
// V rows in 16-byte chunks (chunk c: key c / (D/8), dims 8*(c % (D/8))).
template <int D, int NW>
struct Stage {
    static constexpr int T = NW * 64;
    static constexpr int NCH = KT * D / 8;          // chunks per tile and tensor
    static constexpr int KCH = (NCH + T - 1) / T;   // per thread
    u32x4 k[KCH], v[KCH];
    int64_t off[KCH];  // element offset of the chunk in the cache (same for K and V)
};

struct RowAddr {
    const int32_t *kv_indices;
    int64_t num_pages, page_stride, slot_stride, head_off;
    int page_base, log2_page, page_mask, kv_len;

    // element offset of key `key` (clamped into the request) of this kv head
    __device__ __forceinline__ int64_t operator()(int key) const
    {
        key = min(key, kv_len - 1);
        int64_t pg = kv_indices[page_base + (key >> log2_page)];
        pg = pg < 0 ? 0 : (pg >= num_pages ? num_pages - 1 : pg);
        return pg * page_stride + int64_t(key & page_mask) * slot_stride + head_off;
    }
};

template <int D, int NW>
__device__ __forceinline__ bool chunk_exists(int c)
{
    using S = Stage<D, NW>;
    return S::NCH % S::T == 0 || c < S::NCH;
}

template <int D, int NW>
__device__ __forceinline__ void stage_offsets(Stage<D, NW> &st, const RowAddr &ra, int k0,
                                              int tid)
{
    using S = Stage<D, NW>;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
        const int c = tid + i * S::T;
        st.off[i] = ra(k0 + c / CPR) + (c % CPR) * 8;
    }
}

// Global -> registers.  Keys at or past kv_len are zero-filled: no unwritten
// slot (whatever its bits, even NaN) ever reaches an MFMA.
template <int D, int NW>
__device__ __forceinline__ void stage_load(Stage<D, NW> &st, const PrefillArgs &a, int k0,
                                           int kv_len, int tid)
{
    using S = Stage<D, NW>;
    constexpr int CPR = D / 8;
    const uint16_t *K = static_cast<const uint16_t *>(a.k);
    const uint16_t *V = static_cast<const uint16_t *>(a.v);
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
        const int c = tid + i * S::T;
        const bool ok = chunk_exists<D, NW>(c) && k0 + c / CPR < kv_len;
        const u32x4 z = {0u, 0u, 0u, 0u};
        st.k[i] = ok ? *reinterpret_cast<const u32x4 *>(K + st.off[i]) : z;
        st.v[i] = ok ? *reinterpret_cast<const u32x4 *>(V + st.off[i]) : z;
    }
}

template <int D, int NW>
__device__ __forceinline__ void stage_store(const Stage<D, NW> &st, PrefillBuf<D> &b, int tid)
{
    using S = Stage<D, NW>;
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
        const int c = tid + i * S::T;
        if (chunk_exists<D, NW>(c)) {
            *reinterpret_cast<u32x4 *>(&b.k[c / CPR][(c % CPR) * 8]) = st.k[i];
            *reinterpret_cast<u32x4 *>(&b.v[c / CPR][(c % CPR) * 8]) = st.v[i];
        }
    }
}

// S^T[32 keys x 32 rows] = K . Q^T for the tile in b.
template <int D>
__device__ __forceinline__ f32x16 qk_tile(const PrefillBuf<D> &b, const bf16x8 (&qf)[D / 16],
                                          int l32, int hw)
{
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&b.k[l32][ks * 16 + hw * 8]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
    }
    return s;
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillArgs a)
{
    constexpr int KSTEPS = D / 16;  // QK k-steps
    constexpr int DT = D / 32;      // O^T dim tiles
    __shared__ __attribute__((aligned(16))) PrefillBuf<D> lds[NBUF];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hw = lane >> 5;
    const int G = 1 << a.log2_group;
    const int n_items = a.ws[kHdrNumItems];
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    const int W = a.window_left;
    const float c = a.scale_log2;

    // transposing-read coordinates of this lane (see PrefillBuf)
    const int tr_key = 4 * hw + ((lane & 15) >> 2);             // + 16*kk (+8)
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // + 32*dt

    RowAddr ra;
    ra.kv_indices = a.kv_indices;
    ra.num_pages = a.num_pages;
    ra.slot_stride = int64_t(a.num_kv_heads) * D;
    ra.page_stride = ra.slot_stride * a.page_size;
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

        // prologue: tiles 0 and 1 in LDS sets 0 and 1, tile 2 in registers,
        // tile 3's rows known
        Stage<D, NW> st;
        if (ntiles > 0) {
            stage_offsets(st, ra, kv_begin, tid);
            stage_load(st, a, kv_begin, kv_len, tid);
            stage_store(st, lds[0], tid);
            if (ntiles > 1) {
                stage_offsets(st, ra, kv_begin + KT, tid);
                stage_load(st, a, kv_begin + KT, kv_len, tid);
                stage_offsets(st, ra, kv_begin + 2 * KT, tid);
                stage_store(st, lds[1], tid);
                if (ntiles > 2) {
                    stage_load(st, a, kv_begin + 2 * KT, kv_len, tid);
                    stage_offsets(st, ra, kv_begin + 3 * KT, tid);
                }
            }
        }
        __syncthreads();
        f32x16 s_cur;
        if (ntiles > 0) s_cur = qk_tile<D>(lds[0], qf, l32, hw);

        int cur = 0;  // LDS set of tile j
        for (int j = 0; j < ntiles; ++j) {
            const int k0 = kv_begin + j * KT;
            const int nxt = cur == NBUF - 1 ? 0 : cur + 1;
            const int nn = nxt == NBUF - 1 ? 0 : nxt + 1;

            // S^T of tile j+1 goes to the matrix cores while this tile's softmax
            // runs on the vector ALUs
            f32x16 s_nxt;
            if (j + 1 < ntiles) s_nxt = qk_tile<D>(lds[nxt], qf, l32, hw);

            // accumulator entry i holds key k0 + 8*(i/4) + 4*hw + i%4 of this row
            f32x16 s = s_cur;
            const bool interior = k0 + KT <= kv_len && (!a.causal || k0 + KT - 1 <= pos0) &&
                                  (W < 0 || k0 >= pos_last - W);
            if (!interior) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 8 * (i >> 2) + 4 * hw + (i & 3);
                    const bool vis = key < kv_len && (!a.causal || key <= p_row) &&
                                     (W < 0 || key >= p_row - W);
                    s[i] = vis ? s[i] : kNegInf;
                }
            }
            float mx = fmaxf(s[0], s[1]);
#pragma unroll
            for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[i], s[i + 1]));
            mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;

            // lazy rescale: keep the running maximum unless some row's grows by
            // more than 2^8 (probabilities then stay below 2^8, exact in fp32
            // and in bf16 range), so most tiles skip the O rescale
            if (__any(mx > m + kRescaleLog2)) {
                const float m_new = fmaxf(m, mx);
                const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m - m_new);
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
                m = m_new;
            }
            const float mu = m == kNegInf ? 0.f : m;
            f32x16 pr;
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                pr[i] = fast_exp2(__builtin_fmaf(s[i], c, -mu));
                rs += pr[i];
            }
            l += rs;

            // O^T += V^T . P^T, two k-steps of 16 keys
            const PrefillBuf<D> &bj = lds[cur];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                f32x8 p8;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) p8[jj] = pr[8 * kk + jj];
                const bf16x8 pb = __builtin_convertvector(p8, bf16x8);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const uint16_t *v0 = &bj.v[16 * kk + tr_key][32 * dt + tr_dim];
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)v0);
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(v0 + 8 * (D + VPAD)));
                    const bf16x8 va = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dt], 0, 0, 0);
                }
            }

            // stage tile j+2 into the free LDS set, start loading tile j+3
            if (j + 2 < ntiles) {
                stage_store(st, lds[nn], tid);
                if (j + 3 < ntiles) {
                    stage_load(st, a, k0 + 3 * KT, kv_len, tid);
                    stage_offsets(st, ra, k0 + 4 * KT, tid);
                }
            }
            __syncthreads();
            s_cur = s_nxt;
            cur = nxt;
        }

        // epilogue: the two half-waves hold disjoint keys of each row
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (row_valid) {
            uint16_t *O = static_cast<uint16_t *>(a.o);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int m0 = 0; m0 < 4; ++m0) {
                    f32x4 v4;
#pragma unroll
                    for (int m1 = 0; m1 < 4; ++m1) v4[m1] = o[dt][4 * m0 + m1] * inv;
                    *reinterpret_cast<bf16x4 *>(O + qrow + dt * 32 + 8 * m0 + 4 * hw) =
                        __builtin_convertvector(v4, bf16x4);
                }
            if (a.lse && hw == 0)
                a.lse[int64_t(q_begin + row_tok) * a.num_qo_heads + hk * G + row_head] =
                    l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
        }
        __syncthreads();  // the next item's prologue overwrites LDS set 0
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

hipError_t launch_prefill_bf16(const PrefillArgs &a, int head_dim, int waves, int grid,
                               hipStream_t s)
{
    if (waves == 8) {
        switch (head_dim) {
        case 64: prefill_bf16_kernel<64, 8><<<grid, 512, 0, s>>>(a); break;
        case 128: prefill_bf16_kernel<128, 8><<<grid, 512, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (head_dim) {
        case 64: prefill_bf16_kernel<64, 4><<<grid, 256, 0, s>>>(a); break;
        case 128: prefill_bf16_kernel<128, 4><<<grid, 256, 0, s>>>(a); break;
        case 256: prefill_bf16_kernel<256, 4><<<grid, 256, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

hipError_t launch_attention_fp32(const PrefillArgs &a, int head_dim, int grid, hipStream_t s)
{
    attention_fp32_kernel<<<grid, kGenericThreads, 0, s>>>(a, head_dim);
    return hipGetLastError();
}

int prefill_bf16_blocks_per_cu(int head_dim, int waves)
{
    int n = 0;
    hipError_t e = hipErrorInvalidValue;
    if (waves == 8) {
        if (head_dim == 64)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<64, 8>, 512, 0);
        else if (head_dim == 128)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<128, 8>, 512, 0);
    } else {
        if (head_dim == 64)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<64, 4>, 256, 0);
        else if (head_dim == 128)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<128, 4>, 256, 0);
        else if (head_dim == 256)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_bf16_kernel<256, 4>, 256, 0);
    }
    return e == hipSuccess ? n : 0;
}

}  // namespace pkvs
