// decode.hip -- split-K online-softmax attention of one decode query per
// sequence over the selected chunks of a paged GQA KV cache, plus the merge.
//
// Source: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (attend only to the kept chunks; the budget is the
// number of KV tokens attended).  The split-K form with a final merge of the
// (max, sum, output) partials is this library's design.
//
// One workgroup (4 waves) per (KV split, KV head, sequence) serves the whole
// GQA group, so every selected K/V page is read from HBM once for all
// H_q/H_kv query heads.  A wave consumes one 16-token segment at a time:
//   * S = K_seg . Q_group^T on the matrix cores (v_mfma_f32_16x16x32_bf16):
//     token rows x 16 (zero-padded) query-head columns.  Each lane loads a
//     contiguous D/4-element slice of its token row (16-byte loads covering
//     the 4 KiB page), and K and Q split the reduction over D the same way, so
//     the pairing needs no particular k order;
//   * online softmax per head in fp32 (log2 domain) straight from the MFMA
//     accumulators (lane = head, 4 tokens per lane);
//   * O^T += V^T . P on the matrix cores (v_mfma_f32_16x16x16_bf16): each lane
//     loads one coalesced 4-byte V word per token, the wave transposes the
//     page through a 5 KiB LDS tile, and P (still in registers, laid out
//     exactly as the B operand needs) is split into bf16 hi + lo parts, so the
//     product keeps ~16 bits of P (relative error ~2^-17).
// Each wave loads its page numbers up front (one per lane, read back with
// readlane) and prefetches the next page unconditionally, so the memory
// counters stay exact and one page is always in flight while the current one
// is consumed.  The 4 waves' partials are merged in LDS; with more than one
// split a small kernel merges the splits (a kernel boundary is the cheap way to
// make the partials of all XCDs visible).  HBM-bound.
//
// float32 caches use the same structure with 16x16x4 f32 MFMAs for S and the
// vector ALU for P . V.
#include "bsa_internal.h"

namespace bsa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kDecWaves = 4;
constexpr int kVtStride = 20;  // uint16 per V^T row: 16 tokens + 8 bytes of padding (conflict-free reads)

template <typename T, int D>
struct DecTraits {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int kSlice = D / 4;                              // K elements per lane per token
    static constexpr int kNW = kSlice * (int)sizeof(T) / 16;          // 16-byte words per K slice
    static constexpr int kVD = D / 64;                                // V elements per lane per token
    static constexpr int kRW = (kVD * (int)sizeof(T) + 3) / 4;        // dwords of V per token per lane
    static constexpr int kDT = D / 16;                                // 16-dim output tiles (bf16 path)
};

// Per-wave LDS region: the V^T tile while consuming pages (bf16), the
// probability / alpha tiles (fp32), and afterwards the wave's output slice.
template <int D, int GP>
constexpr int region_floats() {
    constexpr int vt = D * kVtStride / 2;         // bf16 V^T tile, in floats
    constexpr int pf = 16 * 16 + 16;              // fp32 path probability + alpha tiles
    constexpr int ob = GP * D;                    // output slice
    constexpr int a = vt > pf ? vt : pf;
    return a > ob ? a : ob;
}

template <typename T, int D, int GP>
struct WaveState {
    float m_run, l_run;
    f32x4 o[DecTraits<T, D>::kBf16 ? D / 16 : 1];   // bf16 path: O^T, lane (head n16, G) has dims 16dt + 4G + i
    float acc[DecTraits<T, D>::kBf16 ? 1 : GP][D / 64];  // fp32 path: lane owns D/64 dims of every head
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

// Online-softmax step shared by both paths: lane holds S[token 4G+i][head n16].
// Returns the rescale factor of the running state; p[] gets the weights.
__device__ __forceinline__ float softmax_step(const f32x4 &s, int valid, float scale_log2, int G, float &m_run,
                                              float (&p)[4]) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (4 * G + i < valid) ? s[i] * scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2f(x[i] - m_use);
    m_run = m_new;
    return alpha;
}

// bf16: one 16-token segment through the matrix cores.  vt is this wave's
// V^T tile; vr holds V[t][D/64 dims of this lane] for the 16 tokens.
template <int D, int GP>
__device__ __forceinline__ void consume_bf16(WaveState<uint16_t, D, GP> &st,
                                             const uint4 (&ks)[DecTraits<uint16_t, D>::kNW],
                                             const uint32_t (&vr)[16][1],
                                             const uint4 (&qb)[DecTraits<uint16_t, D>::kNW], int valid,
                                             float scale_log2, uint16_t *vt, int lane) {
    constexpr int DT = D / 16;
    const int n16 = lane & 15, G = lane >> 4;
    // V^T tile: row d holds the 16 tokens' V[.][d], two tokens per dword
    wave_lds_sync();  // the previous segment's reads of the tile are done
#pragma unroll
    for (int t = 0; t < 16; t += 4) {
        const uint32_t a = vr[t][0], b = vr[t + 1][0], c = vr[t + 2][0], d = vr[t + 3][0];
        if constexpr (D == 128) {
            const uint2 r0 = make_uint2((a & 0xffffu) | (b << 16), (c & 0xffffu) | (d << 16));
            const uint2 r1 = make_uint2((a >> 16) | (b & 0xffff0000u), (c >> 16) | (d & 0xffff0000u));
            *reinterpret_cast<uint2 *>(vt + (2 * lane) * kVtStride + t) = r0;
            *reinterpret_cast<uint2 *>(vt + (2 * lane + 1) * kVtStride + t) = r1;
        } else {
            *reinterpret_cast<uint2 *>(vt + lane * kVtStride + t) =
                make_uint2((a & 0xffffu) | (b << 16), (c & 0xffffu) | (d << 16));
        }
    }
    const f32x4 s = qk_mfma<uint16_t, D>(ks, qb);
    float p[4];
    const float alpha = softmax_step(s, valid, scale_log2, G, st.m_run, p);
    // P as the B operand: lane (head n16, group G) supplies tokens 4G..4G+3,
    // split into bf16 hi + lo
    uint16_t hi[4], lo[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hi[i] = f32_to_bf16_rne(p[i]);
        lo[i] = f32_to_bf16_rne(p[i] - bf16_to_f32(hi[i]));
        psum += bf16_to_f32(hi[i]) + bf16_to_f32(lo[i]);
    }
    st.l_run = st.l_run * alpha + psum;
    const s16x4 bh = {(short)hi[0], (short)hi[1], (short)hi[2], (short)hi[3]};
    const s16x4 bl = {(short)lo[0], (short)lo[1], (short)lo[2], (short)lo[3]};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.o[dt] *= alpha;
    wave_lds_sync();  // the tile is complete
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const s16x4 a = *reinterpret_cast<const s16x4 *>(vt + (16 * dt + n16) * kVtStride + 4 * G);
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bh, st.o[dt], 0, 0, 0);
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, st.o[dt], 0, 0, 0);
    }
}

// float32: S on the matrix cores, P . V on the vector ALU with P broadcast
// through the wave's LDS tile.
template <int D, int GP>
__device__ __forceinline__ void consume_f32(WaveState<float, D, GP> &st, const uint4 (&ks)[DecTraits<float, D>::kNW],
                                            const uint32_t (&vr)[16][DecTraits<float, D>::kRW],
                                            const uint4 (&qb)[DecTraits<float, D>::kNW], int valid, float scale_log2,
                                            float *pbuf, int lane) {
    constexpr int VD = D / 64;
    const int n16 = lane & 15, G = lane >> 4;
    float *abuf = pbuf + 256;
    const f32x4 s = qk_mfma<float, D>(ks, qb);
    float p[4];
    const float alpha = softmax_step(s, valid, scale_log2, G, st.m_run, p);
    st.l_run = st.l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
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
#pragma unroll
            for (int dd = 0; dd < VD; ++dd) v[dd] = __uint_as_float(vr[4 * t4 + tt][dd]);
#pragma unroll
            for (int j = 0; j < GP; ++j) {
                const float pv = tt == 0 ? pj[j].x : tt == 1 ? pj[j].y : tt == 2 ? pj[j].z : pj[j].w;
#pragma unroll
                for (int dd = 0; dd < VD; ++dd) st.acc[j][dd] = fmaf(pv, v[dd], st.acc[j][dd]);
            }
        }
    }
}

template <typename T, int D, int GP>
__device__ __forceinline__ void consume(WaveState<T, D, GP> &st, const uint4 (&ks)[DecTraits<T, D>::kNW],
                                        const uint32_t (&vr)[16][DecTraits<T, D>::kRW],
                                        const uint4 (&qb)[DecTraits<T, D>::kNW], int valid, float scale_log2,
                                        float *region, int lane) {
    if constexpr (DecTraits<T, D>::kBf16)
        consume_bf16<D, GP>(st, ks, vr, qb, valid, scale_log2, reinterpret_cast<uint16_t *>(region), lane);
    else
        consume_f32<D, GP>(st, ks, vr, qb, valid, scale_log2, region, lane);
}

template <typename T, int D, int GP>
__device__ __forceinline__ void init_state(WaveState<T, D, GP> &st) {
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    if constexpr (DecTraits<T, D>::kBf16) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
        for (int j = 0; j < GP; ++j)
#pragma unroll
            for (int dd = 0; dd < D / 64; ++dd) st.acc[j][dd] = 0.f;
    }
}

// Merge the 4 waves' states in LDS (each wave's output slice reuses its own
// region, which no other wave touches) and write either the final output
// (one split) or this split's partial (unnormalised o, max m, sum l).
template <typename T, int D, int GP>
__device__ __forceinline__ void finish_workgroup(WaveState<T, D, GP> &st, float *regions, float *mbuf, float *lbuf,
                                                 int g, int hq, int b, int h, int split, int splits,
                                                 float *__restrict__ out, float *__restrict__ part_o,
                                                 float *__restrict__ part_ml) {
    constexpr int R = region_floats<D, GP>();
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, G = lane >> 4;
    float l1 = st.l_run + __shfl_xor(st.l_run, 16, 64);
    l1 += __shfl_xor(l1, 32, 64);
    wave_lds_sync();  // this wave's last reads of its region are done
    float *ob = regions + w * R;
    if (G == 0) {
        mbuf[w * 16 + n16] = st.m_run;
        lbuf[w * 16 + n16] = l1;
    }
    if constexpr (DecTraits<T, D>::kBf16) {
        if (n16 < g) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                *reinterpret_cast<float4 *>(ob + n16 * D + 16 * dt + 4 * G) =
                    make_float4(st.o[dt][0], st.o[dt][1], st.o[dt][2], st.o[dt][3]);
        }
    } else {
        constexpr int VD = D / 64;
#pragma unroll
        for (int j = 0; j < GP; ++j)
#pragma unroll
            for (int dd = 0; dd < VD; ++dd) ob[j * D + VD * lane + dd] = st.acc[j][dd];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < g * D; idx += kDecWaves * 64) {
        const int j = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) M = fmaxf(M, mbuf[ww * 16 + j]);
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
            const float mw = mbuf[ww * 16 + j];
            const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
            o = fmaf(f, regions[ww * R + j * D + d], o);
            l = fmaf(f, lbuf[ww * 16 + j], l);
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

// Fixed 16-token pages: one item = one page.
template <typename T, int D, int GP>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 3 : 1) void decode_paged16_kernel(const T *__restrict__ q, int hq, KvView kv,
                                                             const int32_t *__restrict__ sel_idx,
                                                             const int32_t *__restrict__ sel_count, int max_sel,
                                                             float scale_log2, int splits, float *__restrict__ out,
                                                             float *__restrict__ part_o, float *__restrict__ part_ml) {
    using Tr = DecTraits<T, D>;
    constexpr int NW = Tr::kNW, RW = Tr::kRW, R = region_floats<D, GP>();
    __shared__ __attribute__((aligned(16))) float regions[kDecWaves * R];
    __shared__ float mbuf[kDecWaves * 16], lbuf[kDecWaves * 16];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n16 = lane & 15, G = lane >> 4;
    const int g = hq / kv.hkv;
    const int L = kv.seq_lens[b];
    const int npages = (L + 15) >> 4;
    const int nitems = sel_idx ? sel_count[(int64_t)b * kv.hkv + h] : npages;
    const int32_t *items = sel_idx ? sel_idx + ((int64_t)b * kv.hkv + h) * max_sel : nullptr;
    const int i0 = (int)((int64_t)split * nitems / splits), i1 = (int)((int64_t)(split + 1) * nitems / splits);

    uint4 qb[NW];
    load_q_operand<T, D>(q, hq, g, b, h, lane, qb);
    WaveState<T, D, GP> st;
    init_state(st);

    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
    const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
    const int32_t *bt = kv.bt ? kv.bt + (int64_t)b * kv.max_pages : nullptr;
    float *region = regions + w * R;

    // This wave's items are i0 + w, i0 + w + 4, ...  Their logical and physical
    // page numbers are loaded up front, one item per lane, and read back with
    // readlane, so no memory wait sits between a page's prefetch and its use.
    const int first = i0 + w;
    const int n_mine = first < i1 ? (i1 - first + kDecWaves - 1) / kDecWaves : 0;
    auto issue = [&](int page, int phys, uint4 (&ks)[NW], uint32_t (&vr)[16][RW], int &valid) {
        valid = min(16, L - 16 * page);
        load_k_slice<T, D>(kb + (int64_t)phys * kv.sp + (int64_t)n16 * kv.st, ks, G);
        const T *vr0 = vb + (int64_t)phys * kv.sp;
        // every slot of a physical page is allocated: load all 16 rows and clear
        // the rows past the sequence end with a select (padding never leaks)
#pragma unroll
        for (int t = 0; t < 16; ++t) load_v_row<T, D>(vr0 + (int64_t)t * kv.st, vr[t], lane);
    };
    auto clear_tail = [&](uint32_t (&vr)[16][RW], int valid) {
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int r = 0; r < RW; ++r) vr[t][r] = t < valid ? vr[t][r] : 0u;
    };
    for (int base = 0; base < n_mine; base += 64) {
        const int cnt = min(64, n_mine - base);
        int my_page = 0, my_phys = 0;
        if (lane < cnt) {
            const int it = first + kDecWaves * (base + lane);
            my_page = items ? items[it] : it;
            my_phys = bt ? bt[my_page] : b * kv.max_pages + my_page;
        }
        uint4 ksA[NW], ksB[NW];
        uint32_t vrA[16][RW], vrB[16][RW];
        int validA, validB = 0;
        // prefetches are unconditional (clamped to the last item): a conditional
        // load would make every later wait drain all outstanding loads
        issue(__builtin_amdgcn_readlane(my_page, 0), __builtin_amdgcn_readlane(my_phys, 0), ksA, vrA, validA);
        for (int j = 0; j < cnt; j += 2) {
            const int jb = min(j + 1, cnt - 1);
            issue(__builtin_amdgcn_readlane(my_page, jb), __builtin_amdgcn_readlane(my_phys, jb), ksB, vrB, validB);
            clear_tail(vrA, validA);
            consume<T, D, GP>(st, ksA, vrA, qb, validA, scale_log2, region, lane);
            if (j + 1 >= cnt) break;
            const int ja = min(j + 2, cnt - 1);
            issue(__builtin_amdgcn_readlane(my_page, ja), __builtin_amdgcn_readlane(my_phys, ja), ksA, vrA, validA);
            clear_tail(vrB, validB);
            consume<T, D, GP>(st, ksB, vrB, qb, validB, scale_log2, region, lane);
        }
    }
    finish_workgroup<T, D, GP>(st, regions, mbuf, lbuf, g, hq, b, h, split, splits, out, part_o, part_ml);
}

// General chunks: variable token intervals, or fixed pages of any power-of-two
// size.  Each chunk is consumed in 16-token segments with per-lane addresses
// (a segment may straddle two pages); only the segment's valid rows are read.
template <typename T, int D, int GP>
__global__ __launch_bounds__(256) void decode_chunked_kernel(const T *__restrict__ q, int hq, KvView kv, ChunkView ch,
                                                             const int32_t *__restrict__ sel_idx,
                                                             const int32_t *__restrict__ sel_count, int max_sel,
                                                             float scale_log2, int splits, float *__restrict__ out,
                                                             float *__restrict__ part_o, float *__restrict__ part_ml) {
    using Tr = DecTraits<T, D>;
    constexpr int NW = Tr::kNW, RW = Tr::kRW, R = region_floats<D, GP>();
    __shared__ __attribute__((aligned(16))) float regions[kDecWaves * R];
    __shared__ float mbuf[kDecWaves * 16], lbuf[kDecWaves * 16];
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
    init_state(st);

    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
    const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
    const int32_t *bt = kv.bt ? kv.bt + (int64_t)b * kv.max_pages : nullptr;
    auto row_of = [&](const T *base, int tok) {
        const int page = tok >> kv.log2page, slot = tok & (kv.page - 1);
        const int64_t phys = bt ? bt[page] : (int64_t)b * kv.max_pages + page;
        return base + phys * kv.sp + (int64_t)slot * kv.st;
    };
    float *region = regions + w * R;
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
            consume<T, D, GP>(st, ks, vr, qb, valid, scale_log2, region, lane);
        }
    }
    finish_workgroup<T, D, GP>(st, regions, mbuf, lbuf, g, hq, b, h, split, splits, out, part_o, part_ml);
}

// Merge of the splits of one (sequence, query head):
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
// One wave per row; lane s handles split s for the weights (splits <= 64).
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(int splits, const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, float *__restrict__ out,
                                                          int hq) {
    constexpr int VD = D / 64;
    __shared__ float wts[64];
    const int j = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int64_t row = (int64_t)b * hq + j;
    const float *ml = part_ml + row * splits * 2;
    const float m = lane < splits ? ml[2 * lane] : -INFINITY;
    const float l = lane < splits ? ml[2 * lane + 1] : 0.f;
    float M = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float f = m == -INFINITY ? 0.f : exp2f(m - M);
    float lw = f * l;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lw += __shfl_xor(lw, o, 64);
    wts[lane] = f;
    __syncthreads();
    float acc[VD];
#pragma unroll
    for (int dd = 0; dd < VD; ++dd) acc[dd] = 0.f;
    const float *po = part_o + row * splits * D + VD * lane;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) {
        const float ws = wts[s];
#pragma unroll
        for (int dd = 0; dd < VD; ++dd) acc[dd] = fmaf(ws, po[(int64_t)s * D + dd], acc[dd]);
    }
    const float inv = 1.0f / lw;
#pragma unroll
    for (int dd = 0; dd < VD; ++dd) out[row * D + VD * lane + dd] = acc[dd] * inv;
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
        launch_decode_t<T, D, 4>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o, part_ml,
                                 s);
    else if (g <= 8)
        launch_decode_t<T, D, 8>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o, part_ml,
                                 s);
    else
        launch_decode_t<T, D, 16>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                  part_ml, s);
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
