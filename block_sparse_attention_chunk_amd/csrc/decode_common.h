// decode_common.h -- the per-wave machinery of the split-K decode kernels
// (decode.hip, select_decode.hip): operand loads, the matrix-core step for
// one 16-token segment, the online softmax, the page pipeline and the
// workgroup merge.  Internal to libbsa.
#pragma once

#include "bsa_internal.h"

#ifndef BSA_DECODE_PD
#define BSA_DECODE_PD 1
#endif

namespace bsa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kDecWaves = 4;

template <typename T, int D>
struct DecTraits {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int kSlice = D / 4;                         // K elements per lane per token
    static constexpr int kNW = kSlice * (int)sizeof(T) / 16;     // 16-byte words per K slice
    // bf16 V: lane (n16, G) holds tokens 4G..4G+3, dims kVPL*n16 .. kVPL*n16 + kVPL - 1
    static constexpr int kVPL = D / 16;
    // f32 V: lane holds dims kVD*lane .. of all 16 tokens
    static constexpr int kVD = D / 64;
    static constexpr int kRowRegs = kBf16 ? kVPL / 2 : kVD;      // dwords per token row per lane
    static constexpr int kVRegs = kBf16 ? 4 * kRowRegs : 16 * kRowRegs;
};

// Per-wave LDS region: the fp32 path's probability / alpha tiles while
// consuming pages, afterwards the wave's output slice.
template <int D, int GP>
constexpr int region_floats() {
    constexpr int pf = 16 * 16 + 16;
    constexpr int ob = GP * D;
    return pf > ob ? pf : ob;
}

template <typename T, int D, int GP>
struct WaveState {
    float m_run, l_run;
    f32x4 o[DecTraits<T, D>::kBf16 ? D / 16 : 1];         // bf16: O^T tiles (see consume_bf16)
    float acc[DecTraits<T, D>::kBf16 ? 1 : GP][D / 64];   // f32: lane owns D/64 dims of every head
};

template <typename T, int D>
__device__ __forceinline__ void load_k_slice(const T *row, uint4 (&ks)[DecTraits<T, D>::kNW], int G) {
    const uint4 *p = reinterpret_cast<const uint4 *>(row + DecTraits<T, D>::kSlice * G);
#pragma unroll
    for (int i = 0; i < DecTraits<T, D>::kNW; ++i) ks[i] = p[i];
}

// One token row's share of V for this lane.
template <typename T, int D>
__device__ __forceinline__ void load_v_row(const T *row, uint32_t *dst, int lane) {
    using Tr = DecTraits<T, D>;
    if constexpr (Tr::kBf16) {
        const T *p = row + Tr::kVPL * (lane & 15);
        if constexpr (Tr::kVPL == 8) {
            const uint4 x = *reinterpret_cast<const uint4 *>(p);
            dst[0] = x.x, dst[1] = x.y, dst[2] = x.z, dst[3] = x.w;
        } else {
            const uint2 x = *reinterpret_cast<const uint2 *>(p);
            dst[0] = x.x, dst[1] = x.y;
        }
    } else if constexpr (Tr::kVD == 2) {
        const uint2 x = *reinterpret_cast<const uint2 *>(row + 2 * lane);
        dst[0] = x.x, dst[1] = x.y;
    } else {
        dst[0] = *reinterpret_cast<const uint32_t *>(row + lane);
    }
}

// Token slot of V row r of this lane (bf16: 4 rows per lane; f32: all 16).
template <typename T, int D>
__device__ __forceinline__ int v_token(int r, int G) {
    return DecTraits<T, D>::kBf16 ? 4 * G + r : r;
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
    mx = max_across_rows16(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2f(x[i] - m_use);
    m_run = m_new;
    return alpha;
}

// A operand of output tile dt: V[token 4G+i][dim kVPL*n16 + dt], i = 0..3,
// taken from the lane's own registers (the k index of the product is the
// token, the row index the dimension).
template <int D>
__device__ __forceinline__ s16x4 v_operand(const uint32_t (&vr)[DecTraits<uint16_t, D>::kVRegs], int dt) {
    constexpr int RR = DecTraits<uint16_t, D>::kRowRegs;
    const int w = dt >> 1;
    const uint32_t r0 = vr[w], r1 = vr[RR + w], r2 = vr[2 * RR + w], r3 = vr[3 * RR + w];
    uint32_t lo, hi;
    if (dt & 1) {
        lo = (r0 >> 16) | (r1 & 0xffff0000u);
        hi = (r2 >> 16) | (r3 & 0xffff0000u);
    } else {
        lo = (r0 & 0xffffu) | (r1 << 16);
        hi = (r2 & 0xffffu) | (r3 << 16);
    }
    return __builtin_bit_cast(s16x4, make_uint2(lo, hi));
}

// bf16: one 16-token segment through the matrix cores.
//   S^T-free form: S = K . Q^T with lane (token n16, group G) supplying the
//   G-th quarter of the token's K row and of every head's q;
//   O^T[d][head] += V^T . P with the output tile dt's row r standing for
//   dim kVPL*r + dt, so each lane's 4 V rows are already the A operand.
template <int D, int GP>
__device__ __forceinline__ void consume_bf16(WaveState<uint16_t, D, GP> &st,
                                             const uint4 (&ks)[DecTraits<uint16_t, D>::kNW],
                                             const uint32_t (&vr)[DecTraits<uint16_t, D>::kVRegs],
                                             const uint4 (&qb)[DecTraits<uint16_t, D>::kNW], int valid,
                                             float scale_log2, int lane) {
    constexpr int DT = D / 16;
    const int G = lane >> 4;
    const f32x4 s = qk_mfma<uint16_t, D>(ks, qb);
    float p[4];
    const float alpha = softmax_step(s, valid, scale_log2, G, st.m_run, p);
    // P as the B operand: lane (head n16, group G) supplies tokens 4G..4G+3,
    // split into bf16 hi + lo (the product keeps ~16 bits of P)
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
    for (int dt = 0; dt < DT; ++dt) {
        const s16x4 a = v_operand<D>(vr, dt);
        st.o[dt] *= alpha;
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bh, st.o[dt], 0, 0, 0);
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, st.o[dt], 0, 0, 0);
    }
}

// float32: S on the matrix cores, P . V on the vector ALU with P broadcast
// through the wave's LDS tile.
template <int D, int GP>
__device__ __forceinline__ void consume_f32(WaveState<float, D, GP> &st, const uint4 (&ks)[DecTraits<float, D>::kNW],
                                            const uint32_t (&vr)[DecTraits<float, D>::kVRegs],
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
            for (int dd = 0; dd < VD; ++dd) v[dd] = __uint_as_float(vr[(4 * t4 + tt) * VD + dd]);
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
                                        const uint32_t (&vr)[DecTraits<T, D>::kVRegs],
                                        const uint4 (&qb)[DecTraits<T, D>::kNW], int valid, float scale_log2,
                                        float *region, int lane) {
    if constexpr (DecTraits<T, D>::kBf16)
        consume_bf16<D, GP>(st, ks, vr, qb, valid, scale_log2, lane);
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
// region, which no other wave touches) and write either the final output of
// the group's heads, rows out_row0 + j (part_o == NULL), or a partial
// (unnormalised o, max m, sum l) to partial rows prow0 + j * pstride.  NT is
// the workgroup size; waves from kDecWaves on hold no state and only help
// with the merge.
template <typename T, int D, int GP, int NT = kDecWaves * 64>
__device__ __forceinline__ void finish_workgroup_at(WaveState<T, D, GP> &st, float *regions, float *mbuf,
                                                    float *lbuf, int g, int64_t out_row0, int64_t prow0, int pstride,
                                                    float *__restrict__ out, float *__restrict__ part_o,
                                                    float *__restrict__ part_ml) {
    constexpr int R = region_floats<D, GP>();
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, G = lane >> 4;
    const float l1 = sum_across_rows16(st.l_run);
    wave_lds_sync();  // this wave's last reads of its region are done
    float *ob = regions + w * R;
    if (w < kDecWaves) {
        if (G == 0) {
            mbuf[w * 16 + n16] = st.m_run;
            lbuf[w * 16 + n16] = l1;
        }
        if constexpr (DecTraits<T, D>::kBf16) {
            // tile dt, row 4G+i holds dim kVPL*(4G+i) + dt of head n16
            constexpr int VPL = DecTraits<T, D>::kVPL;
            if (n16 < g) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int d4 = 0; d4 < VPL; d4 += 4)
                        *reinterpret_cast<float4 *>(ob + n16 * D + VPL * (4 * G + i) + d4) =
                            make_float4(st.o[d4][i], st.o[d4 + 1][i], st.o[d4 + 2][i], st.o[d4 + 3][i]);
            }
        } else {
            constexpr int VD = D / 64;
#pragma unroll
            for (int j = 0; j < GP; ++j)
#pragma unroll
                for (int dd = 0; dd < VD; ++dd) ob[j * D + VD * lane + dd] = st.acc[j][dd];
        }
    }
    __syncthreads();
    // each thread merges 4 consecutive dims of one head
    constexpr int D4 = D / 4;
    for (int idx = threadIdx.x; idx < g * D4; idx += NT) {
        const int j = idx / D4, d = (idx % D4) * 4;
        float mw[kDecWaves], M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
            mw[ww] = mbuf[ww * 16 + j];
            M = fmaxf(M, mw[ww]);
        }
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        float l = 0.f;
#pragma unroll
        for (int ww = 0; ww < kDecWaves; ++ww) {
            const float f = mw[ww] == -INFINITY ? 0.f : exp2f(mw[ww] - M);
            const float4 r = *reinterpret_cast<const float4 *>(regions + ww * R + j * D + d);
            o.x = fmaf(f, r.x, o.x);
            o.y = fmaf(f, r.y, o.y);
            o.z = fmaf(f, r.z, o.z);
            o.w = fmaf(f, r.w, o.w);
            l = fmaf(f, lbuf[ww * 16 + j], l);
        }
        if (!part_o) {
            const int64_t row = out_row0 + j;
            *reinterpret_cast<float4 *>(out + row * D + d) = make_float4(o.x / l, o.y / l, o.z / l, o.w / l);
        } else {
            const int64_t prow = prow0 + (int64_t)j * pstride;
            *reinterpret_cast<float4 *>(part_o + prow * D + d) = o;
            if (d == 0) *reinterpret_cast<float2 *>(part_ml + prow * 2) = make_float2(M, l);
        }
    }
}

// The split-K destination: split `split` of (sequence b, KV head h); the
// partials are laid out [batch][H_q][splits] (part_o is NULL for one split).
template <typename T, int D, int GP, int NT = kDecWaves * 64>
__device__ __forceinline__ void finish_workgroup(WaveState<T, D, GP> &st, float *regions, float *mbuf, float *lbuf,
                                                 int g, int hq, int b, int h, int split, int splits,
                                                 float *__restrict__ out, float *__restrict__ part_o,
                                                 float *__restrict__ part_ml) {
    const int64_t row0 = (int64_t)b * hq + h * g;
    finish_workgroup_at<T, D, GP, NT>(st, regions, mbuf, lbuf, g, row0, row0 * splits + split, splits, out, part_o,
                                      part_ml);
}

// Merge of the splits of one (sequence, query head) row:
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
// One wave; lane s holds split s's (m, l) (splits <= 64) and every lane owns
// D/64 output dims.  All loads of a batch of 32 splits are issued before the
// first use (clamped to the last split), so the wave waits on memory once per
// batch.
template <int D>
__device__ __forceinline__ void merge_split_row(int splits, const float *__restrict__ part_o,
                                                const float *__restrict__ part_ml, float *__restrict__ out,
                                                int64_t row, int lane) {
    constexpr int VD = D / 64, SB = 32;
    const float2 ml = reinterpret_cast<const float2 *>(part_ml + row * splits * 2)[min(lane, splits - 1)];
    const float ml_m = ml.x, ml_l = ml.y;
    const float *po = part_o + row * splits * D + VD * lane;
    float f = 0.f, lw = 0.f, acc[VD];
#pragma unroll
    for (int dd = 0; dd < VD; ++dd) acc[dd] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += SB) {
        float ov[SB][VD];
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            const float *p = po + (int64_t)min(s0 + i, splits - 1) * D;
            if constexpr (VD == 2) {
                const float2 x = *reinterpret_cast<const float2 *>(p);
                ov[i][0] = x.x, ov[i][1] = x.y;
            } else {
                ov[i][0] = p[0];
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the batch is in flight before the first wait
        if (s0 == 0) {
            const float m = lane < splits ? ml_m : -INFINITY;
            const float M = wave_max_all(m);
            f = m == -INFINITY ? 0.f : exp2f(m - M);
            lw = wave_sum_all(lane < splits ? f * ml_l : 0.f);
        }
        // split s's weight sits in lane s (0 for lanes >= splits)
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), min(s0 + i, 63)));
            const bool use = s0 + i < splits;
#pragma unroll
            for (int dd = 0; dd < VD; ++dd) acc[dd] = use ? fmaf(ws, ov[i][dd], acc[dd]) : acc[dd];
        }
    }
    const float inv = 1.0f / lw;
    if constexpr (VD == 2) {
        reinterpret_cast<float2 *>(out + row * D)[lane] = make_float2(acc[0] * inv, acc[1] * inv);
    } else {
        out[row * D + lane] = acc[0] * inv;
    }
}

template <typename T, int D>
__device__ __forceinline__ void load_q_operand(const T *__restrict__ q, int hq, int g, int b, int h, int lane,
                                               uint4 (&qb)[DecTraits<T, D>::kNW]) {
    const int n16 = lane & 15, G = lane >> 4;
    // unconditional (padding columns read a real head and are masked), so the
    // load never sits in a branch that would force a full memory wait
    load_k_slice<T, D>(q + ((int64_t)b * hq + h * g + min(n16, g - 1)) * D, qb, G);
    const uint32_t m = n16 < g ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < DecTraits<T, D>::kNW; ++i) {
        qb[i].x &= m;
        qb[i].y &= m;
        qb[i].z &= m;
        qb[i].w &= m;
    }
}

// Streams this wave's n_mine items (whole 16-token pages of one (sequence,
// KV head)) through consume().  page_of(base) gives lane l the logical page of
// the wave's item base + l and phys_of(base, page) its physical page; both are
// called once per 64 items for every lane, and only lanes
// l < min(64, n_mine - base) are used.  Page numbers are held one
// item per lane and read back with readlane, so no memory wait sits between a
// page's prefetch and its use; prefetches are unconditional (clamped to the
// last item), because a conditional load would make every later wait drain all
// outstanding loads.  PD pages are in flight while the current one is
// consumed.
template <typename T, int D, int GP, int PD, typename PageOf, typename PhysOf>
__device__ __forceinline__ void stream_pages(WaveState<T, D, GP> &st, const uint4 (&qb)[DecTraits<T, D>::kNW],
                                             const KvView &kv, const T *kb, const T *vb, int L, int n_mine,
                                             PageOf page_of, PhysOf phys_of, float scale_log2, float *region,
                                             int lane) {
    using Tr = DecTraits<T, D>;
    constexpr int NW = Tr::kNW, VR = Tr::kVRegs, NB = PD + 1;
    const int n16 = lane & 15, G = lane >> 4;
    auto issue = [&](int page, int phys, uint4 (&ks)[NW], uint32_t (&vr)[VR], int &valid) {
        valid = min(16, L - 16 * page);
        load_k_slice<T, D>(kb + (int64_t)phys * kv.sp + (int64_t)n16 * kv.st, ks, G);
        const T *v0 = vb + (int64_t)phys * kv.sp;
        // every slot of a physical page is allocated: load all rows and clear
        // the rows past the sequence end with a select (padding never leaks)
#pragma unroll
        for (int r = 0; r < VR / Tr::kRowRegs; ++r)
            load_v_row<T, D>(v0 + (int64_t)v_token<T, D>(r, G) * kv.st, vr + r * Tr::kRowRegs, lane);
    };
    auto clear_tail = [&](uint32_t (&vr)[VR], int valid) {
#pragma unroll
        for (int r = 0; r < VR / Tr::kRowRegs; ++r)
#pragma unroll
            for (int c = 0; c < Tr::kRowRegs; ++c)
                vr[r * Tr::kRowRegs + c] = v_token<T, D>(r, G) < valid ? vr[r * Tr::kRowRegs + c] : 0u;
    };
    for (int base = 0; base < n_mine; base += 64) {
        const int cnt = min(64, n_mine - base);
        const int pg = page_of(base);
        int my_page = 0, my_phys = 0;
        if (lane < cnt) {
            my_page = pg;
            my_phys = phys_of(base, pg);
        }
        uint4 ks[NB][NW];
        uint32_t vr[NB][VR];
        int valid[NB];
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            const int jj = min(s, cnt - 1);
            issue(__builtin_amdgcn_readlane(my_page, jj), __builtin_amdgcn_readlane(my_phys, jj), ks[s], vr[s],
                  valid[s]);
        }
        // whole rounds of NB items, then the (up to PD) items still in flight;
        // no early exit inside a round, so the counter waits stay exact
        const int full = cnt - cnt % NB;
        for (int j = 0; j < full; j += NB) {
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                const int jn = min(j + s + PD, cnt - 1);
                const int sn = (s + PD) % NB;
                issue(__builtin_amdgcn_readlane(my_page, jn), __builtin_amdgcn_readlane(my_phys, jn), ks[sn], vr[sn],
                      valid[sn]);
                // keep the prefetch ahead of the consumption: the scheduler
                // would otherwise sink these loads next to their use
                __builtin_amdgcn_sched_barrier(0);
                clear_tail(vr[s], valid[s]);
                consume<T, D, GP>(st, ks[s], vr[s], qb, valid[s], scale_log2, region, lane);
            }
        }
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (full + s < cnt) {
                clear_tail(vr[s], valid[s]);
                consume<T, D, GP>(st, ks[s], vr[s], qb, valid[s], scale_log2, region, lane);
            }
        }
    }
}

}  // namespace bsa
