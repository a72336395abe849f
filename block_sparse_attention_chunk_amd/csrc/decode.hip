// decode.hip -- split-K online-softmax attention of one decode query per
// sequence over the selected chunks of a paged GQA KV cache, plus the merge.
//
// Source: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (attend only to the kept chunks; the budget is the
// number of KV tokens attended).  The split-K form with a final merge of the
// (max, sum, output) partials is this library's design.
//
// Layout of the work: one workgroup (4 waves) per (KV split, KV head,
// sequence) serves the whole GQA group, so every selected K/V page is read
// from HBM once for all H_q/H_kv query heads.  A wave processes one 16-token
// segment at a time:
//   * S = K_seg . Q_group^T on the matrix cores: the 16 token rows are the
//     MFMA rows, the (zero-padded) 16 query heads the columns; each lane loads
//     a contiguous D/4-element slice of its token row (coalesced 16-byte
//     loads; the whole 4 KiB page per wave) and the reduction over D is split
//     the same way for K and Q, so the pairing needs no particular k order;
//   * online softmax per head in fp32 (log2 domain), p broadcast through a
//     per-wave LDS tile;
//   * O += P . V on the vector ALU: each lane owns D/64 output dims of every
//     head and reads V rows with one coalesced load per token.
// Pages are double-buffered so the next page's 8 KiB are in flight while the
// current one is consumed.  The 4 waves' partials are merged in LDS; with
// more than one split a second kernel merges the splits.  HBM-bound.
#include "bsa_internal.h"

namespace bsa {

constexpr int kDecWaves = 4;

template <typename T, int D>
struct DecTraits {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int kSlice = D / 4;                              // K elements per lane per token
    static constexpr int kNW = kSlice * (int)sizeof(T) / 16;          // 16-byte words per K slice
    static constexpr int kSteps = kBf16 ? kSlice / 8 : kSlice;        // MFMA steps over D
    static constexpr int kVD = D / 64;                                // output dims per lane
    static constexpr int kRW = (kVD * (int)sizeof(T) + 3) / 4;        // dwords of V per token per lane
};

template <typename T, int D>
struct QOperand {
    using Tr = DecTraits<T, D>;
    uint4 w[Tr::kNW];
};

template <typename T, int D, int GP>
struct WaveState {
    float m_run, l_run;
    float acc[GP][D / 64];
};

template <typename T, int D>
__device__ __forceinline__ void load_k_slice(const T *row, uint4 (&ks)[DecTraits<T, D>::kNW], int G) {
    const uint4 *p = reinterpret_cast<const uint4 *>(row + DecTraits<T, D>::kSlice * G);
#pragma unroll
    for (int i = 0; i < DecTraits<T, D>::kNW; ++i) ks[i] = p[i];
}

template <typename T, int D>
__device__ __forceinline__ void load_v_row(const T *row, uint32_t (&vr)[DecTraits<T, D>::kRW], int lane) {
    using Tr = DecTraits<T, D>;
    if constexpr (Tr::kBf16 && Tr::kVD == 2) {
        vr[0] = *reinterpret_cast<const uint32_t *>(row + 2 * lane);
    } else if constexpr (Tr::kBf16) {
        vr[0] = *reinterpret_cast<const uint16_t *>(row + lane);
    } else if constexpr (Tr::kVD == 2) {
        const uint2 x = *reinterpret_cast<const uint2 *>(row + 2 * lane);
        vr[0] = x.x;
        vr[1] = x.y;
    } else {
        vr[0] = *reinterpret_cast<const uint32_t *>(row + lane);
    }
}

template <typename T, int D>
__device__ __forceinline__ void v_to_float(const uint32_t (&vr)[DecTraits<T, D>::kRW], float (&v)[D / 64]) {
    using Tr = DecTraits<T, D>;
    if constexpr (Tr::kBf16 && Tr::kVD == 2) {
        v[0] = bf16_lo(vr[0]);
        v[1] = bf16_hi(vr[0]);
    } else if constexpr (Tr::kBf16) {
        v[0] = bf16_lo(vr[0]);
    } else {
#pragma unroll
        for (int i = 0; i < Tr::kVD; ++i) v[i] = __uint_as_float(vr[i]);
    }
}

template <typename T, int D>
__device__ __forceinline__ f32x4 qk_mfma(const uint4 (&ks)[DecTraits<T, D>::kNW],
                                         const uint4 (&qb)[DecTraits<T, D>::kNW]) {
    using Tr = DecTraits<T, D>;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Tr::kBf16) {
#pragma unroll
        for (int i = 0; i < Tr::kNW; ++i)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ks[i]),
                                                        __builtin_bit_cast(bf16x8, qb[i]), s, 0, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < Tr::kNW; ++i) {
            const uint32_t a[4] = {ks[i].x, ks[i].y, ks[i].z, ks[i].w};
            const uint32_t bq[4] = {qb[i].x, qb[i].y, qb[i].z, qb[i].w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[c]), __uint_as_float(bq[c]), s, 0, 0, 0);
        }
    }
    return s;
}

// Consume one 16-token segment: `valid` leading tokens are real.  pbuf / abuf
// are this wave's LDS tiles ([16 heads][16 tokens] probabilities, [16] alphas).
template <typename T, int D, int GP>
__device__ __forceinline__ void consume_segment(WaveState<T, D, GP> &st, const uint4 (&ks)[DecTraits<T, D>::kNW],
                                                const uint32_t (&vr)[16][DecTraits<T, D>::kRW],
                                                const uint4 (&qb)[DecTraits<T, D>::kNW], int valid,
                                                float scale_log2, float *pbuf, float *abuf, int lane) {
    constexpr int VD = D / 64;
    const int n16 = lane & 15, G = lane >> 4;
    const f32x4 s = qk_mfma<T, D>(ks, qb);
    // lane holds S[token 4G+i][head n16]
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * G + i < valid) ? s[i] * scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(st.m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(st.m_run - m_use);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2f(x[i] - m_use);
    st.l_run = st.l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    st.m_run = m_new;
    wave_lds_sync();
    if (n16 < GP) {
        *reinterpret_cast<float4 *>(pbuf + n16 * 16 + 4 * G) = make_float4(p[0], p[1], p[2], p[3]);
        if (G == 0) abuf[n16] = alpha;
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < GP; ++j) {
        const float a = abuf[j];
#pragma unroll
        for (int dd = 0; dd < VD; ++dd) st.acc[j][dd] *= a;
    }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
        float4 pj[GP];
#pragma unroll
        for (int j = 0; j < GP; ++j) pj[j] = *reinterpret_cast<const float4 *>(pbuf + j * 16 + 4 * t4);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            float v[VD];
            v_to_float<T, D>(vr[4 * t4 + tt], v);
#pragma unroll
            for (int j = 0; j < GP; ++j) {
                const float pv = tt == 0 ? pj[j].x : tt == 1 ? pj[j].y : tt == 2 ? pj[j].z : pj[j].w;
#pragma unroll
                for (int dd = 0; dd < VD; ++dd) st.acc[j][dd] = fmaf(pv, v[dd], st.acc[j][dd]);
            }
        }
    }
}

// Merge the 4 waves' states in LDS and write either the final output
// (one split) or this split's partial (unnormalised o, max m, sum l).
template <typename T, int D, int GP>
__device__ __forceinline__ void finish_workgroup(WaveState<T, D, GP> &st, float *obuf, float *mbuf, float *lbuf,
                                                 int g, int hq, int b, int h, int split, int splits,
                                                 float *__restrict__ out, float *__restrict__ part_o,
                                                 float *__restrict__ part_ml) {
    constexpr int VD = D / 64;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, G = lane >> 4;
    float l1 = st.l_run + __shfl_xor(st.l_run, 16, 64);
    l1 += __shfl_xor(l1, 32, 64);
    if (G == 0 && n16 < GP) {
        mbuf[w * GP + n16] = st.m_run;
        lbuf[w * GP + n16] = l1;
    }
#pragma unroll
    for (int j = 0; j < GP; ++j)
#pragma unroll
        for (int dd = 0; dd < VD; ++dd) obuf[(w * GP + j) * D + VD * lane + dd] = st.acc[j][dd];
    __syncthreads();
    for (int idx = threadIdx.x; idx < g * D; idx += kDecWaves * 64) {
        const int j = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, mbuf[ww * GP + j]);
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
            const float mw = mbuf[ww * GP + j];
            const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
            o = fmaf(f, obuf[(ww * GP + j) * D + d], o);
            l = fmaf(f, lbuf[ww * GP + j], l);
        }
        const int64_t row = (int64_t)b * hq + h * g + j;
        if (splits == 1) {
            out[row * D + d] = o / l;
        } else {
            part_o[(row * splits + split) * D + d] = o;
            if (d == 0) {
                part_ml[(row * splits + split) * 2] = M;
                part_ml[(row * splits + split) * 2 + 1] = l;
            }
        }
    }
}

template <typename T, int D>
__device__ __forceinline__ void load_q_operand(const T *__restrict__ q, int hq, int g, int b, int h, int lane,
                                               uint4 (&qb)[DecTraits<T, D>::kNW]) {
    const int n16 = lane & 15, G = lane >> 4;
    if (n16 < g) {
        load_k_slice<T, D>(q + ((int64_t)b * hq + h * g + n16) * D, qb, G);
    } else {
#pragma unroll
        for (int i = 0; i < DecTraits<T, D>::kNW; ++i) qb[i] = make_uint4(0, 0, 0, 0);
    }
}

// Fixed 16-token pages: one item = one page; the page's physical address is
// wave-uniform and pages are double-buffered.
template <typename T, int D, int GP>
__global__ __launch_bounds__(256) void decode_paged16_kernel(const T *__restrict__ q, int hq, KvView kv,
                                                             const int32_t *__restrict__ sel_idx,
                                                             const int32_t *__restrict__ sel_count, int max_sel,
                                                             float scale_log2, int splits, float *__restrict__ out,
                                                             float *__restrict__ part_o, float *__restrict__ part_ml) {
    using Tr = DecTraits<T, D>;
    constexpr int NW = Tr::kNW, RW = Tr::kRW;
    __shared__ __attribute__((aligned(16))) float pbuf[kDecWaves][16 * 16];
    __shared__ float abuf[kDecWaves][16];
    __shared__ __attribute__((aligned(16))) float obuf[kDecWaves * GP * D];
    __shared__ float mbuf[kDecWaves * GP], lbuf[kDecWaves * GP];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n16 = lane & 15;
    const int g = hq / kv.hkv;
    const int L = kv.seq_lens[b];
    const int npages = (L + 15) >> 4;
    const int nitems = sel_idx ? sel_count[(int64_t)b * kv.hkv + h] : npages;
    const int32_t *items = sel_idx ? sel_idx + ((int64_t)b * kv.hkv + h) * max_sel : nullptr;
    const int i0 = (int)((int64_t)split * nitems / splits), i1 = (int)((int64_t)(split + 1) * nitems / splits);

    uint4 qb[NW];
    load_q_operand<T, D>(q, hq, g, b, h, lane, qb);
    WaveState<T, D, GP> st;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
#pragma unroll
    for (int j = 0; j < GP; ++j)
#pragma unroll
        for (int dd = 0; dd < D / 64; ++dd) st.acc[j][dd] = 0.f;

    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
    const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
    const int32_t *bt = kv.bt ? kv.bt + (int64_t)b * kv.max_pages : nullptr;
    const int G = lane >> 4;

    auto page_of = [&](int i) {
        return __builtin_amdgcn_readfirstlane(items ? items[i] : i);
    };
    auto load_page = [&](int page, uint4 (&ks)[NW], uint32_t (&vr)[16][RW], int &valid) {
        const int64_t phys = bt ? bt[page] : (int64_t)b * kv.max_pages + page;
        valid = min(16, L - 16 * page);
        const T *kr = kb + phys * kv.sp + (int64_t)n16 * kv.st;
        load_k_slice<T, D>(kr, ks, G);
        const T *vr0 = vb + phys * kv.sp;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            if (t < valid) {
                load_v_row<T, D>(vr0 + (int64_t)t * kv.st, vr[t], lane);
            } else {
#pragma unroll
                for (int r = 0; r < RW; ++r) vr[t][r] = 0u;
            }
        }
    };

    float *pb = pbuf[w];
    float *ab = abuf[w];
    int it = i0 + w;
    if (it < i1) {
        uint4 ksA[NW], ksB[NW];
        uint32_t vrA[16][RW], vrB[16][RW];
        int validA, validB = 0;
        load_page(page_of(it), ksA, vrA, validA);
        while (true) {
            const int itB = it + kDecWaves;
            if (itB < i1) load_page(page_of(itB), ksB, vrB, validB);
            consume_segment<T, D, GP>(st, ksA, vrA, qb, validA, scale_log2, pb, ab, lane);
            if (itB >= i1) break;
            const int itA = itB + kDecWaves;
            if (itA < i1) load_page(page_of(itA), ksA, vrA, validA);
            consume_segment<T, D, GP>(st, ksB, vrB, qb, validB, scale_log2, pb, ab, lane);
            if (itA >= i1) break;
            it = itA;
        }
    }
    finish_workgroup<T, D, GP>(st, obuf, mbuf, lbuf, g, hq, b, h, split, splits, out, part_o, part_ml);
}

// General chunks: variable token intervals, or fixed pages of any power-of-two
// size.  Each chunk is consumed in 16-token segments with per-lane addresses
// (a segment may straddle two pages).
template <typename T, int D, int GP>
__global__ __launch_bounds__(256) void decode_chunked_kernel(const T *__restrict__ q, int hq, KvView kv, ChunkView ch,
                                                             const int32_t *__restrict__ sel_idx,
                                                             const int32_t *__restrict__ sel_count, int max_sel,
                                                             float scale_log2, int splits, float *__restrict__ out,
                                                             float *__restrict__ part_o, float *__restrict__ part_ml) {
    using Tr = DecTraits<T, D>;
    constexpr int NW = Tr::kNW, RW = Tr::kRW;
    __shared__ __attribute__((aligned(16))) float pbuf[kDecWaves][16 * 16];
    __shared__ float abuf[kDecWaves][16];
    __shared__ __attribute__((aligned(16))) float obuf[kDecWaves * GP * D];
    __shared__ float mbuf[kDecWaves * GP], lbuf[kDecWaves * GP];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n16 = lane & 15, G = lane >> 4;
    const int g = hq / kv.hkv;
    const int L = kv.seq_lens[b];
    const int nch = ch.starts ? ch.num[b] : (L + kv.page - 1) >> kv.log2page;
    const int nitems = sel_idx ? sel_count[(int64_t)b * kv.hkv + h] : nch;
    const int32_t *items = sel_idx ? sel_idx + ((int64_t)b * kv.hkv + h) * max_sel : nullptr;
    const int i0 = (int)((int64_t)split * nitems / splits), i1 = (int)((int64_t)(split + 1) * nitems / splits);

    uint4 qb[NW];
    load_q_operand<T, D>(q, hq, g, b, h, lane, qb);
    WaveState<T, D, GP> st;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
#pragma unroll
    for (int j = 0; j < GP; ++j)
#pragma unroll
        for (int dd = 0; dd < D / 64; ++dd) st.acc[j][dd] = 0.f;

    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
    const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
    const int32_t *bt = kv.bt ? kv.bt + (int64_t)b * kv.max_pages : nullptr;
    auto row_of = [&](const T *base, int tok) {
        const int page = tok >> kv.log2page, slot = tok & (kv.page - 1);
        const int64_t phys = bt ? bt[page] : (int64_t)b * kv.max_pages + page;
        return base + phys * kv.sp + (int64_t)slot * kv.st;
    };
    float *pb = pbuf[w];
    float *ab = abuf[w];
    for (int it = i0 + w; it < i1; it += kDecWaves) {
        const int c = __builtin_amdgcn_readfirstlane(items ? items[it] : it);
        int s, e;
        if (ch.starts) {
            s = ch.starts[(int64_t)b * (ch.max_chunks + 1) + c];
            e = ch.starts[(int64_t)b * (ch.max_chunks + 1) + c + 1];
        } else {
            s = c << kv.log2page;
            e = min(s + kv.page, L);
        }
        for (int t0 = s; t0 < e; t0 += 16) {
            const int valid = min(16, e - t0);
            uint4 ks[NW];
            uint32_t vr[16][RW];
            if (n16 < valid) {
                load_k_slice<T, D>(row_of(kb, t0 + n16), ks, G);
            } else {
#pragma unroll
                for (int i = 0; i < NW; ++i) ks[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                if (t < valid) {
                    load_v_row<T, D>(row_of(vb, t0 + t), vr[t], lane);
                } else {
#pragma unroll
                    for (int r = 0; r < RW; ++r) vr[t][r] = 0u;
                }
            }
            consume_segment<T, D, GP>(st, ks, vr, qb, valid, scale_log2, pb, ab, lane);
        }
    }
    finish_workgroup<T, D, GP>(st, obuf, mbuf, lbuf, g, hq, b, h, split, splits, out, part_o, part_ml);
}

// Merge of the splits: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(int splits, const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, float *__restrict__ out,
                                                          int hq) {
    constexpr int VD = D / 64;
    const int j = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int64_t row = (int64_t)b * hq + j;
    const float *ml = part_ml + row * splits * 2;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[2 * s]);
    float o[VD], l = 0.f;
#pragma unroll
    for (int dd = 0; dd < VD; ++dd) o[dd] = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float m = ml[2 * s];
        const float f = m == -INFINITY ? 0.f : exp2f(m - M);
        l = fmaf(f, ml[2 * s + 1], l);
        const float *po = part_o + (row * splits + s) * D + VD * lane;
#pragma unroll
        for (int dd = 0; dd < VD; ++dd) o[dd] = fmaf(f, po[dd], o[dd]);
    }
#pragma unroll
    for (int dd = 0; dd < VD; ++dd) out[row * D + VD * lane + dd] = o[dd] / l;
}

template <typename T, int D, int GP>
static void launch_decode_t(const void *q, int hq, const KvView &kv, const ChunkView &ch, const int32_t *sel_idx,
                            const int32_t *sel_count, int max_sel, float scale_log2, int splits, float *out,
                            float *part_o, float *part_ml, hipStream_t s) {
    dim3 grid(splits, kv.hkv, kv.batch), block(kDecWaves * 64);
    if (!ch.starts && kv.page == 16)
        hipLaunchKernelGGL((decode_paged16_kernel<T, D, GP>), grid, block, 0, s, (const T *)q, hq, kv, sel_idx,
                           sel_count, max_sel, scale_log2, splits, out, part_o, part_ml);
    else
        hipLaunchKernelGGL((decode_chunked_kernel<T, D, GP>), grid, block, 0, s, (const T *)q, hq, kv, ch, sel_idx,
                           sel_count, max_sel, scale_log2, splits, out, part_o, part_ml);
}

template <typename T, int D>
static void launch_decode_g(const void *q, int hq, const KvView &kv, const ChunkView &ch, const int32_t *sel_idx,
                            const int32_t *sel_count, int max_sel, float scale_log2, int splits, float *out,
                            float *part_o, float *part_ml, hipStream_t s) {
    const int g = hq / kv.hkv;
    if (g <= 4)
        launch_decode_t<T, D, 4>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o, part_ml, s);
    else if (g <= 8)
        launch_decode_t<T, D, 8>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o, part_ml, s);
    else
        launch_decode_t<T, D, 16>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o, part_ml,
                                  s);
}

hipError_t launch_decode(const void *q, int32_t hq, const KvView &kv, const ChunkView &ch, const int32_t *sel_idx,
                         const int32_t *sel_count, int32_t max_sel, float scale, int32_t splits, float *out, void *ws,
                         hipStream_t s) {
    const float scale_log2 = scale * kLog2e;
    float *part_o = nullptr, *part_ml = nullptr;
    if (splits > 1) {
        part_o = (float *)ws;
        part_ml = part_o + (size_t)kv.batch * hq * splits * kv.d;
    }
    if (kv.dtype == BSA_BF16) {
        if (kv.d == 128)
            launch_decode_g<uint16_t, 128>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                           part_ml, s);
        else
            launch_decode_g<uint16_t, 64>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                          part_ml, s);
    } else {
        if (kv.d == 128)
            launch_decode_g<float, 128>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                        part_ml, s);
        else
            launch_decode_g<float, 64>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                       part_ml, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    dim3 grid(hq, kv.batch);
    if (kv.d == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(64), 0, s, splits, part_o, part_ml, out, hq);
    else
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(64), 0, s, splits, part_o, part_ml, out, hq);
    return hipGetLastError();
}

}  // namespace bsa
