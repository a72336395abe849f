// score.hip -- chunk scoring against the current query (decode) and against
// query tiles (prefill).
//
// Source: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (envelope = per-dimension min/max upper bound,
// centroid = mean of chunk keys); "Technische Samenvatting ... Blok-schaarse
// Aandacht", section "Methodologie" steps 1-2 (the tile score is the maximum
// over the tile's query rows).  Selection is per KV head, so the scores of a
// GQA group's query heads are combined by their maximum.
#include "lds_dma.h"

namespace bsa {

// ---------------------------------------------------------------------------
// Decode: one thread per chunk, the GQA group's query in LDS.
// Envelope per head: sum_d max(q*kmin, q*kmax) = sum_d (q+ * kmax + q- * kmin)
// with q+ = max(q, 0), q- = min(q, 0): two FMAs per element, one of them a
// multiply by an exact zero, so each term is rounded once.  HBM-bound on the
// metadata read (512 B per chunk and KV head at d = 128).
// ---------------------------------------------------------------------------
template <typename T, int D, int GP, int KIND>
__global__ __launch_bounds__(256) void score_decode_kernel(const T *__restrict__ q, int hq, KvView kv, ChunkView ch,
                                                           const T *__restrict__ kmin, const T *__restrict__ kmax,
                                                           const float *__restrict__ cen, float *__restrict__ out) {
    constexpr int NQ = KIND == BSA_ENVELOPE ? 2 * GP : GP;  // floats per dim in LDS
    __shared__ float qs[D * NQ];
    const int h = blockIdx.y, b = blockIdx.z;
    const int g = hq / kv.hkv;
    for (int i = threadIdx.x; i < D * GP; i += blockDim.x) {
        const int d = i / GP, j = i % GP;
        float x = 0.f;
        if (j < g) {
            const T *qr = q + ((int64_t)b * hq + h * g + j) * D + d;
            if constexpr (sizeof(T) == 2)
                x = bf16_to_f32(*reinterpret_cast<const uint16_t *>(qr));
            else
                x = *reinterpret_cast<const float *>(qr);
        }
        if constexpr (KIND == BSA_ENVELOPE) {
            qs[d * NQ + j] = fmaxf(x, 0.f);
            qs[d * NQ + GP + j] = fminf(x, 0.f);
        } else {
            qs[d * NQ + j] = x;
        }
    }
    __syncthreads();
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= ch.max_chunks) return;
    const int n = ch.starts ? ch.num[b] : (kv.seq_lens[b] + kv.page - 1) >> kv.log2page;
    const int64_t orow = ((int64_t)b * kv.hkv + h) * ch.max_chunks + c;
    if (c >= n) {
        out[orow] = -INFINITY;
        return;
    }
    float acc[GP];
#pragma unroll
    for (int j = 0; j < GP; ++j) acc[j] = 0.f;
    const int64_t mrow = orow * D;
    if constexpr (KIND == BSA_ENVELOPE) {
        constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte load
        const uint4 *pmin = reinterpret_cast<const uint4 *>(kmin + mrow);
        const uint4 *pmax = reinterpret_cast<const uint4 *>(kmax + mrow);
#pragma unroll 2
        for (int v = 0; v < D / EPV; ++v) {
            const uint4 wmin = pmin[v], wmax = pmax[v];
            float lo[EPV], hi[EPV];
            if constexpr (sizeof(T) == 2) {
                const uint32_t a[4] = {wmin.x, wmin.y, wmin.z, wmin.w}, bb[4] = {wmax.x, wmax.y, wmax.z, wmax.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo[2 * i] = bf16_lo(a[i]);
                    lo[2 * i + 1] = bf16_hi(a[i]);
                    hi[2 * i] = bf16_lo(bb[i]);
                    hi[2 * i + 1] = bf16_hi(bb[i]);
                }
            } else {
                lo[0] = __uint_as_float(wmin.x); lo[1] = __uint_as_float(wmin.y);
                lo[2] = __uint_as_float(wmin.z); lo[3] = __uint_as_float(wmin.w);
                hi[0] = __uint_as_float(wmax.x); hi[1] = __uint_as_float(wmax.y);
                hi[2] = __uint_as_float(wmax.z); hi[3] = __uint_as_float(wmax.w);
            }
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const float *qd = qs + (v * EPV + e) * NQ;
#pragma unroll
                for (int j = 0; j < GP; ++j) {
                    acc[j] = fmaf(qd[j], hi[e], acc[j]);
                    acc[j] = fmaf(qd[GP + j], lo[e], acc[j]);
                }
            }
        }
    } else {
        const float4 *pc = reinterpret_cast<const float4 *>(cen + mrow);
#pragma unroll 4
        for (int v = 0; v < D / 4; ++v) {
            const float4 w = pc[v];
            const float cv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float *qd = qs + (v * 4 + e) * NQ;
#pragma unroll
                for (int j = 0; j < GP; ++j) acc[j] = fmaf(qd[j], cv[e], acc[j]);
            }
        }
    }
    float best = acc[0];
#pragma unroll
    for (int j = 1; j < GP; ++j)
        if (j < g) best = fmaxf(best, acc[j]);
    out[orow] = best;
}

// max(a, b) as one instruction: fmaxf would first quiet both inputs (the
// compiler cannot prove matrix-core results or lane moves quiet), doubling the
// row reduction's vector work.  Operands here are scores or -inf, never NaN.
__device__ __forceinline__ float max_nn(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Maximum over the 16 lanes of each 16-lane row (rotations inside the row).
__device__ __forceinline__ float row16_max(float v) {
    v = max_nn(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));  // row_ror:8
    v = max_nn(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));  // row_ror:4
    v = max_nn(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));  // row_ror:2
    v = max_nn(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));  // row_ror:1
    return v;
}

// Decode on the matrix cores (bf16 caches): one wave scores 16 chunks for the
// whole GQA group.  S[chunk][head] = sum_f A[chunk][f] * B[f][head] over 2*D
// features: envelope A = [kmax | kmin], B = [q+ ; q-] (q+ and q- are exact in
// bf16, so every product is exact and only the fp32 accumulation rounds);
// centroid A = [c_hi | c_lo] with the fp32 centroid split into two bf16
// terms, B = [q ; q].  The group maximum is a 16-lane max over the MFMA
// columns.  Per chunk this reads the 512-byte metadata row once and issues a
// handful of instructions, so the kernel stays on the HBM roof for any group
// size (a vector-ALU form needs 2*g*D FMAs per 512 bytes, at the ridge for
// g = 8).
__device__ __forceinline__ uint4 split_sign(uint4 w, bool neg);

template <int D, int KIND>
__global__ __launch_bounds__(256) void score_decode_mfma_kernel(const uint16_t *__restrict__ q, int hq, KvView kv,
                                                                ChunkView ch, const uint16_t *__restrict__ kmin,
                                                                const uint16_t *__restrict__ kmax,
                                                                const float *__restrict__ cen,
                                                                float *__restrict__ out) {
    constexpr int NS = 2 * D / 32;  // MFMA steps over 2*D features
    args_ready(q, hq, kv.hkv, kv.seq_lens, kv.page, kv.log2page, ch.starts, ch.num, ch.max_chunks, kmin, kmax, cen,
               out);
    const int h = blockIdx.y, b = blockIdx.z;
    const int g = hq / kv.hkv;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, G = lane >> 4;
    float *orow = out + ((int64_t)b * kv.hkv + h) * ch.max_chunks;
    const int64_t mbase = ((int64_t)b * kv.hkv + h) * ch.max_chunks * D;
    const int stride = gridDim.x * 4;
    const int n_groups = (ch.max_chunks + 15) / 16;
    const int first = blockIdx.x * 4 + w;
    if (first >= n_groups) return;
    // The row length, the query and the first metadata group are requested
    // together: every load is unconditional and none depends on another.
    const int *len_src = ch.starts ? ch.num : kv.seq_lens;
    const int len = len_src[b];
    bf16x8 bq[NS];
    uint4 qv[NS / 2];
    {
        const int jq = min(n16, g - 1);  // padding columns load a real head, zeroed below
#pragma unroll
        for (int s = 0; s < NS / 2; ++s)
            qv[s] = *reinterpret_cast<const uint4 *>(q + ((int64_t)b * hq + h * g + jq) * D + 32 * s + 8 * G);
    }
    // rows are clamped into the allocated max_chunks, not to the row length, so
    // the first requests do not wait for it; chunks past the length within the
    // last live group are scored and discarded
    auto load = [&](int grp, uint4 (&a)[NS]) {
        const int c = min(grp * 16 + n16, ch.max_chunks - 1);
        const int64_t mrow = mbase + (int64_t)c * D;
        if constexpr (KIND == BSA_ENVELOPE) {
#pragma unroll
            for (int s = 0; s < NS / 2; ++s) {
                a[s] = *reinterpret_cast<const uint4 *>(kmax + mrow + 32 * s + 8 * G);
                a[s + NS / 2] = *reinterpret_cast<const uint4 *>(kmin + mrow + 32 * s + 8 * G);
            }
        } else {
#pragma unroll
            for (int s = 0; s < NS / 2; ++s) {
                const float4 x0 = *reinterpret_cast<const float4 *>(cen + mrow + 32 * s + 8 * G);
                const float4 x1 = *reinterpret_cast<const float4 *>(cen + mrow + 32 * s + 8 * G + 4);
                a[s] = make_uint4(__float_as_uint(x0.x), __float_as_uint(x0.y), __float_as_uint(x0.z),
                                  __float_as_uint(x0.w));
                a[s + NS / 2] = make_uint4(__float_as_uint(x1.x), __float_as_uint(x1.y), __float_as_uint(x1.z),
                                           __float_as_uint(x1.w));
            }
        }
    };
    uint4 aA[NS], aB[NS];
    load(first, aA);
    // the length is used only from here on, so its wait follows every request
    // above (the compiler would otherwise compute the chunk count, and wait,
    // before issuing them)
    int len_v = len;
    asm volatile("" : "+v"(len_v)::"memory");
    const int n = ch.starts ? len_v : (len_v + kv.page - 1) >> kv.log2page;
    {
        const uint32_t qm = n16 < g ? 0xffffffffu : 0u;  // a mask: a select would move the loads into a branch
#pragma unroll
        for (int s = 0; s < NS / 2; ++s) {
            qv[s].x &= qm;
            qv[s].y &= qm;
            qv[s].z &= qm;
            qv[s].w &= qm;
        }
#pragma unroll
        for (int s = 0; s < NS / 2; ++s) {
            if constexpr (KIND == BSA_ENVELOPE) {
                bq[s] = __builtin_bit_cast(bf16x8, split_sign(qv[s], false));
                bq[s + NS / 2] = __builtin_bit_cast(bf16x8, split_sign(qv[s], true));
            } else {
                bq[s] = __builtin_bit_cast(bf16x8, qv[s]);
                bq[s + NS / 2] = bq[s];
            }
        }
    }
    // chunk groups of 16: wave-strided over the grid, the next group's metadata
    // in flight while the current one is reduced
    auto score = [&](int grp, const uint4 (&araw)[NS]) {
        const int c0 = grp * 16;
        uint4 a[NS];
        if constexpr (KIND == BSA_ENVELOPE) {
#pragma unroll
            for (int s = 0; s < NS; ++s) a[s] = araw[s];
        } else {
            // fp32 centroid -> bf16 hi + lo
#pragma unroll
            for (int s = 0; s < NS / 2; ++s) {
                const uint32_t xw[8] = {araw[s].x, araw[s].y, araw[s].z, araw[s].w,
                                        araw[s + NS / 2].x, araw[s + NS / 2].y, araw[s + NS / 2].z,
                                        araw[s + NS / 2].w};
                uint16_t hi[8], lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = __uint_as_float(xw[e]);
                    hi[e] = f32_to_bf16_rne(x);
                    lo[e] = f32_to_bf16_rne(x - bf16_to_f32(hi[e]));
                }
                a[s] = make_uint4(hi[0] | (uint32_t(hi[1]) << 16), hi[2] | (uint32_t(hi[3]) << 16),
                                  hi[4] | (uint32_t(hi[5]) << 16), hi[6] | (uint32_t(hi[7]) << 16));
                a[s + NS / 2] = make_uint4(lo[0] | (uint32_t(lo[1]) << 16), lo[2] | (uint32_t(lo[3]) << 16),
                                           lo[4] | (uint32_t(lo[5]) << 16), lo[6] | (uint32_t(lo[7]) << 16));
            }
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s]), bq[s], acc, 0, 0, 0);
        // lane holds S[chunk 4G+i][head n16]; maximum over the group's heads
        float m[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = n16 < g ? acc[i] : -INFINITY;
            v = row16_max(v);
            m[i] = v;
        }
        if (n16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int cc = c0 + 4 * G + i;
                if (cc < ch.max_chunks) orow[cc] = cc < n ? m[i] : -INFINITY;
            }
        }
    };
    // only the groups holding the row's chunks are read; the slots past them
    // (up to max_chunks) get -inf without a load
    const int n_live = min((n + 15) >> 4, n_groups);
    int grp = first;
    for (; grp < n_live; grp += 2 * stride) {
        load(min(grp + stride, n_live - 1), aB);   // unconditional: exact memory counters
        score(grp, aA);
        if (grp + stride >= n_live) {
            grp += stride;
            break;
        }
        load(min(grp + 2 * stride, n_live - 1), aA);
        score(grp + stride, aB);
    }
    for (; grp < n_groups; grp += stride) {
        const int cc = grp * 16 + lane;
        if (lane < 16 && cc < ch.max_chunks) orow[cc] = -INFINITY;
    }
}

template <typename T, int D, int KIND>
static void dispatch_decode_g(const void *q, int hq, const KvView &kv, const ChunkView &ch, const void *kmin,
                              const void *kmax, const float *cen, float *scores, hipStream_t s) {
    const int g = hq / kv.hkv;
    dim3 grid((ch.max_chunks + 255) / 256, kv.hkv, kv.batch), block(256);
    const T *qq = (const T *)q;
    const T *mn = (const T *)kmin;
    const T *mx = (const T *)kmax;
    if (g <= 4)
        hipLaunchKernelGGL((score_decode_kernel<T, D, 4, KIND>), grid, block, 0, s, qq, hq, kv, ch, mn, mx, cen, scores);
    else if (g <= 8)
        hipLaunchKernelGGL((score_decode_kernel<T, D, 8, KIND>), grid, block, 0, s, qq, hq, kv, ch, mn, mx, cen, scores);
    else
        hipLaunchKernelGGL((score_decode_kernel<T, D, 16, KIND>), grid, block, 0, s, qq, hq, kv, ch, mn, mx, cen,
                           scores);
}

template <typename T, int D>
static void dispatch_decode_kind(const void *q, int hq, const KvView &kv, const ChunkView &ch, const void *kmin,
                                 const void *kmax, const float *cen, int kind, float *scores, hipStream_t s) {
    if (kind == BSA_ENVELOPE)
        dispatch_decode_g<T, D, BSA_ENVELOPE>(q, hq, kv, ch, kmin, kmax, cen, scores, s);
    else
        dispatch_decode_g<T, D, BSA_CENTROID>(q, hq, kv, ch, kmin, kmax, cen, scores, s);
}

hipError_t launch_score_decode(const void *q, int32_t hq, const KvView &kv, const ChunkView &ch, const void *kmin,
                               const void *kmax, const float *cen, int32_t kind, float *scores, hipStream_t s) {
    if (kv.dtype == BSA_BF16) {
        // About eight 16-chunk groups per wave (q is loaded once per wave and
        // the next group is in flight while one is reduced), but at least one
        // workgroup per compute unit in all and at most one group per wave:
        // one group per wave at one sequence, eight per wave at 16 x 32K tokens
        // (measured: 13.2 us there against 14.6 us with four per wave and
        // 15.4 us with a second group in flight).
        const int n_groups = (ch.max_chunks + 15) / 16;
        const int bh = kv.batch * kv.hkv;
        int gx = (n_groups + 31) / 32;
        const int fill = (256 + bh - 1) / bh;
        if (gx < fill) gx = fill;
        if (gx > (n_groups + 3) / 4) gx = (n_groups + 3) / 4;
        dim3 grid(gx, kv.hkv, kv.batch), block(256);
        const uint16_t *qq = (const uint16_t *)q, *mn = (const uint16_t *)kmin, *mx = (const uint16_t *)kmax;
        if (kv.d == 128) {
            if (kind == BSA_ENVELOPE)
                hipLaunchKernelGGL((score_decode_mfma_kernel<128, BSA_ENVELOPE>), grid, block, 0, s, qq, hq, kv, ch, mn,
                                   mx, cen, scores);
            else
                hipLaunchKernelGGL((score_decode_mfma_kernel<128, BSA_CENTROID>), grid, block, 0, s, qq, hq, kv, ch, mn,
                                   mx, cen, scores);
        } else {
            if (kind == BSA_ENVELOPE)
                hipLaunchKernelGGL((score_decode_mfma_kernel<64, BSA_ENVELOPE>), grid, block, 0, s, qq, hq, kv, ch, mn,
                                   mx, cen, scores);
            else
                hipLaunchKernelGGL((score_decode_mfma_kernel<64, BSA_CENTROID>), grid, block, 0, s, qq, hq, kv, ch, mn,
                                   mx, cen, scores);
        }
    } else {
        if (kv.d == 128) dispatch_decode_kind<float, 128>(q, hq, kv, ch, kmin, kmax, cen, kind, scores, s);
        else dispatch_decode_kind<float, 64>(q, hq, kv, ch, kmin, kmax, cen, kind, scores, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Query tiles on the matrix cores.  One workgroup per (tile t, KV head h).
// The group's G query heads x 64 rows form 4G row tiles of 16 rows, dealt
// round-robin to NW = min(8, 4G) waves (wave w takes row tiles w, w + NW,
// ...).  Waves w and w + 4 share a SIMD, so each SIMD carries G row tiles'
// worth of matrix work (with one wave per head and G = 7 the busiest SIMD
// would carry 8 of an average 7).  The block scores of a head form the product
//     S^T[block][row] = sum_f A[block][f] * B[f][row]
// over 2*D features: envelope A = [kmax | kmin], B = [q+ ; q-];
// centroid A = [c_hi | c_lo] (float32 centroid split into two bf16 terms),
// B = [q ; q].  bf16 inputs, fp32 accumulation (v_mfma_f32_16x16x32_bf16).
// Every row of the group shares the K metadata (GQA), so a wave may mix heads.
// A wave's rows are reduced by max in registers and across the 16 lanes of a
// row group, the waves through LDS.  Metadata for 16 blocks is staged in LDS
// and shared by all waves.
// ---------------------------------------------------------------------------
constexpr int kTileRows = 64;
constexpr int kBlkTile = 16;               // blocks per MFMA row tile

__device__ __forceinline__ uint4 split_sign(uint4 w, bool neg) {
    // keep the bf16 halves whose sign matches (neg: negative halves, else the rest)
    uint32_t in[4] = {w.x, w.y, w.z, w.w}, o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t spread = ((in[i] & 0x80008000u) >> 15) * 0xffffu;
        o[i] = neg ? (in[i] & spread) : (in[i] & ~spread);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Staging of metadata tiles (16 blocks x 512 bytes: envelope [kmax | kmin]
// bf16, centroid fp32) straight from global memory into an LDS ring,
// kStStages tiles deep.  Wave instruction u of a tile (8 of 1 KiB) fills block
// rows 2u, 2u+1; lane l writes 16-byte slot l mod 32 of its row, and fetches
// the logical chunk slot ^ (row mod 16), so the 16 rows one MFMA operand read
// touches (same logical chunk) sit at 16 different 16-byte positions of the
// 256-byte bank line: a 16-lane read is free of bank conflicts.
constexpr int kStRowBytes = 512;
constexpr int kStTileBytes = kBlkTile * kStRowBytes;
constexpr int kStStages = 6;
constexpr int kStInstrs = kStTileBytes / 1024;

__device__ __forceinline__ int st_slot(int row, int chunk) { return chunk ^ (row & 15); }

template <int G>
struct TileWaves {
    static constexpr int NRT = 4 * G;                  // row tiles of the group
    static constexpr int NW = NRT < 8 ? NRT : 8;       // waves
    static constexpr int HI = (NRT + NW - 1) / NW;     // row tiles of waves w < NRT % NW (all, if 0)
    static constexpr int LO = NRT / NW;
    static constexpr int NI = (kStInstrs + NW - 1) / NW;  // staging instructions per wave and tile
};

struct TileScoreArgs {
    const uint16_t *q;
    int hq, rows;
    KvView kv;
    int n_blocks;
    const uint16_t *kmin, *kmax;
    const float *cen;
    int causal;
    float *out;
};

// One wave's part of a workgroup, for a wave that holds CNT row tiles.  Per
// 16-block tile: wait for this wave's copies of it, one barrier, request the
// tile kStStages - 1 ahead into the buffer everyone has just finished, then
// the tile's 8 * CNT MFMAs, with the previous tile's row maxima (vector ALU)
// interleaved so the matrix and vector units work at the same time; the
// waves' maxima of the tile before are combined after the next barrier.  Every
// wave passes the same barriers, whatever its CNT.  No compiler-visible load
// sits in the loop.  Tiles are taken in descending order, the causal ones with
// the most blocks first.
template <int KIND, int G, int CNT>
__device__ __forceinline__ void score_tiles_wave(const TileScoreArgs &A, char *ring, float (*red)[8][kBlkTile]) {
    using TW = TileWaves<G>;
    constexpr int D = 128, PF = kStStages, NW = TW::NW, NI = TW::NI;
    const int t = gridDim.x - 1 - blockIdx.x, h = blockIdx.y;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n16 = lane & 15, G4 = lane >> 4;
    const int r0 = t * kTileRows;
    const int vis = A.causal ? min(A.n_blocks, (min(r0 + kTileRows, A.rows) - 1) / A.kv.page + 1) : A.n_blocks;
    float *orow = A.out + ((int64_t)t * A.kv.hkv + h) * A.n_blocks;
    const int64_t mbase = ((int64_t)h * A.n_blocks) * D;  // batch 1
    const int ntiles16 = (vis + kBlkTile - 1) / kBlkTile;

    // B operand: this wave's row tiles (row tile j: query head h*G + j/4,
    // rows 16*(j%4) ..), 8 k-steps of 32 features
    bf16x8 bq[CNT][8];
    bool rvalid[CNT];
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
        const int j = w + NW * i;
        const int r = r0 + (j & 3) * 16 + n16;
        rvalid[i] = r < A.rows;
        const uint32_t m = rvalid[i] ? 0xffffffffu : 0u;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v = *reinterpret_cast<const uint4 *>(A.q + ((int64_t)min(r, A.rows - 1) * A.hq + h * G + (j >> 2)) * D +
                                                       32 * s + 8 * G4);
            v.x &= m, v.y &= m, v.z &= m, v.w &= m;
            if constexpr (KIND == BSA_ENVELOPE) {
                bq[i][s] = __builtin_bit_cast(bf16x8, split_sign(v, false));
                bq[i][s + 4] = __builtin_bit_cast(bf16x8, split_sign(v, true));
            } else {
                bq[i][s] = __builtin_bit_cast(bf16x8, v);
                bq[i][s + 4] = bq[i][s];
            }
        }
    }
    wait_vmcnt<0>();  // the query is in registers before any copy is issued

    // this wave's share of tile bt into ring buffer `stage`; tiles past the
    // last one reload the last one (they land in a buffer nobody reads)
    auto issue = [&](int bt, int stage) {
        bt = min(bt, ntiles16 - 1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int u = min(w + NW * i, kStInstrs - 1);  // duplicates rewrite identical bytes
            const int row = 2 * u + (lane >> 5);
            const int c = st_slot(row, lane & 31);
            const int blk = min(bt * kBlkTile + row, vis - 1);
            const char *src;
            if constexpr (KIND == BSA_ENVELOPE)
                src = reinterpret_cast<const char *>((c < 16 ? A.kmax : A.kmin) + mbase + (int64_t)blk * D +
                                                     8 * (c & 15));
            else
                src = reinterpret_cast<const char *>(A.cen + mbase + (int64_t)blk * D + 4 * c);
            dma16(src, lds_addr(ring) + stage * kStTileBytes + u * 1024);
        }
    };
    // the waves' maxima of tile bt -> the output row (wave 0, lanes 0..15)
    auto finalize = [&](int bt) {
        if (threadIdx.x < kBlkTile) {
            const int blk = bt * kBlkTile + threadIdx.x;
            if (blk < vis) {
                float m = red[bt & 1][0][threadIdx.x];
#pragma unroll
                for (int j = 1; j < NW; ++j) m = fmaxf(m, red[bt & 1][j][threadIdx.x]);
                orow[blk] = m;
            }
        }
    };

    auto mma = [&](int stage, f32x4 (&acc)[CNT]) {
        const char *fb = ring + stage * kStTileBytes + n16 * kStRowBytes;
#pragma unroll
        for (int i = 0; i < CNT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (KIND == BSA_ENVELOPE) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(fb + 16 * st_slot(n16, 4 * s + G4));
#pragma unroll
                for (int i = 0; i < CNT; ++i)
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq[i][s], acc[i], 0, 0, 0);
            }
        } else {
            // fp32 centroid dims 32s + 8G4 .. +8 -> bf16 hi (step s) and lo (step s + 4)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float4 x0 = *reinterpret_cast<const float4 *>(fb + 16 * st_slot(n16, 8 * s + 2 * G4));
                const float4 x1 = *reinterpret_cast<const float4 *>(fb + 16 * st_slot(n16, 8 * s + 2 * G4 + 1));
                const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                uint16_t hi[8], lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    hi[e] = f32_to_bf16_rne(x[e]);
                    lo[e] = f32_to_bf16_rne(x[e] - bf16_to_f32(hi[e]));
                }
                const uint4 ah = make_uint4(hi[0] | (uint32_t(hi[1]) << 16), hi[2] | (uint32_t(hi[3]) << 16),
                                            hi[4] | (uint32_t(hi[5]) << 16), hi[6] | (uint32_t(hi[7]) << 16));
                const uint4 al = make_uint4(lo[0] | (uint32_t(lo[1]) << 16), lo[2] | (uint32_t(lo[3]) << 16),
                                            lo[4] | (uint32_t(lo[5]) << 16), lo[6] | (uint32_t(lo[7]) << 16));
#pragma unroll
                for (int i = 0; i < CNT; ++i) {
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah), bq[i][s], acc[i],
                                                                     0, 0, 0);
                    acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al), bq[i][s + 4],
                                                                     acc[i], 0, 0, 0);
                }
            }
        }
    };
    // lane holds S^T[block 4G4+e][row n16] of each row tile: maximum over the
    // wave's rows -> this wave's slot of the tile's maxima
    auto reduce = [&](const f32x4 (&acc)[CNT], int bt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < CNT; ++i) m = max_nn(m, rvalid[i] ? acc[i][e] : -INFINITY);
            m = row16_max(m);
            red[bt & 1][w][4 * G4 + e] = m;  // every lane of the row holds the same maximum
        }
    };
    // the MFMAs of one tile and the row reduction of the previous one in a
    // single scheduling region, interleaved: one MFMA, then two vector ops
    auto interleave = [&]() {
#pragma unroll
        for (int k = 0; k < 8 * CNT; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
    };
    int cur = 0;  // ring buffer of the next tile
    auto top = [&](int bt) {
        wait_vmcnt<(PF - 2) * NI>();  // this wave's copies of tile bt have landed
        wait_lgkm0();
        stage_barrier();  // every wave's copies too; the previous tile's buffer and maxima are free
        issue(bt + PF - 1, cur == 0 ? PF - 1 : cur - 1);
        if (bt >= 2) finalize(bt - 2);
    };

#pragma unroll
    for (int p = 0; p < PF - 1; ++p) issue(p, p);
    f32x4 accA[CNT], accB[CNT];
    int bt = 0;
    for (; bt + 1 < ntiles16; bt += 2) {
        top(bt);
        mma(cur, accA);
        if (bt > 0) {
            reduce(accB, bt - 1);
            interleave();
        }
        cur = cur == PF - 1 ? 0 : cur + 1;
        top(bt + 1);
        mma(cur, accB);
        reduce(accA, bt);
        interleave();
        cur = cur == PF - 1 ? 0 : cur + 1;
    }
    if (bt < ntiles16) {  // an odd count: the last tile goes to accA
        top(bt);
        mma(cur, accA);
        if (bt > 0) reduce(accB, bt - 1);
        reduce(accA, bt);
    } else {
        reduce(accB, bt - 1);
    }
    wait_vmcnt<0>();  // no copy may still target LDS when the workgroup ends
    wait_lgkm0();
    stage_barrier();
    if (ntiles16 >= 2) finalize(ntiles16 - 2);
    finalize(ntiles16 - 1);
    for (int blk = vis + threadIdx.x; blk < A.n_blocks; blk += 64 * NW) orow[blk] = -INFINITY;
}

template <int KIND, int G>
__global__ __launch_bounds__(64 * TileWaves<G>::NW) void score_tiles_kernel(TileScoreArgs A) {
    using TW = TileWaves<G>;
    __shared__ __attribute__((aligned(1024))) char ring[kStStages * kStTileBytes];
    __shared__ float red[2][8][kBlkTile];
    args_ready(A.q, A.hq, A.rows, A.kv.hkv, A.kv.page, A.n_blocks, A.kmin, A.kmax, A.cen, A.causal, A.out);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (TW::HI == TW::LO || w < TW::NRT % TW::NW)
        score_tiles_wave<KIND, G, TW::HI>(A, ring, red);
    else
        score_tiles_wave<KIND, G, TW::LO>(A, ring, red);
}

hipError_t launch_score_tiles(const void *q, int32_t hq, int32_t rows, int32_t tile_rows, const KvView &kv,
                              int32_t n_blocks, const void *kmin, const void *kmax, const float *cen, int32_t kind,
                              int32_t causal, float *scores, hipStream_t s) {
    (void)tile_rows;  // validated to be 64 by the caller
    const int g = hq / kv.hkv;
    const int n_tiles = (rows + kTileRows - 1) / kTileRows;
    const TileScoreArgs A{(const uint16_t *)q, hq, rows, kv, n_blocks, (const uint16_t *)kmin, (const uint16_t *)kmax,
                          cen, causal, scores};
    dim3 grid(n_tiles, kv.hkv);
#define BSA_ST(G)                                                                                                   \
    case G:                                                                                                         \
        if (kind == BSA_ENVELOPE)                                                                                   \
            hipLaunchKernelGGL((score_tiles_kernel<BSA_ENVELOPE, G>), grid, dim3(64 * TileWaves<G>::NW), 0, s, A);  \
        else                                                                                                        \
            hipLaunchKernelGGL((score_tiles_kernel<BSA_CENTROID, G>), grid, dim3(64 * TileWaves<G>::NW), 0, s, A);  \
        break;
    switch (g) {
        BSA_ST(1) BSA_ST(2) BSA_ST(3) BSA_ST(4) BSA_ST(5) BSA_ST(6) BSA_ST(7) BSA_ST(8)
    default:
        return hipErrorInvalidValue;
    }
#undef BSA_ST
    return hipGetLastError();
}

}  // namespace bsa
