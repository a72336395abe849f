// meta.hip -- per-chunk key metadata (min / max envelope and centroid).
//
// Source: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (method table: envelope = per-dimension min/max of
// a chunk's keys, centroid = mean of a chunk's keys); "Technische Samenvatting
// ... Blok-schaarse Aandacht", section "Methodologie" step 1.
//
// One wave per (sequence, KV head, chunk).  A lane reads 16 bytes of a token
// row (8 bf16 or 4 fp32 dimensions), so one wave instruction covers 64 / NG
// whole rows (NG lanes per row) and every lane issues a few wide loads instead
// of one narrow load per token.  Lane (j, dg) takes tokens s + j, s + j + TPW,
// ... of dimension group dg; the partial min / max / sum of the TPW lanes of a
// dimension group are then combined with in-row rotations and the gfx950 row
// swaps.  With fixed pages a chunk is one page, whose physical number is read
// once; variable chunks may cross pages, so each lane looks its token's page
// up.  min / max are exact; the centroid is a float32 sum (per lane in token
// order, then a tree over the TPW lanes) divided by the token count.
// HBM-bound: one read of K, 1/8 (bf16 envelope) of it written back.  The same
// kernel refreshes only the chunks that newly appended tokens touched (update
// mode), with results identical to a full rebuild of those chunks.
#include "bsa_internal.h"

namespace bsa {

// Update mode (max_touched > 0): wave i of a sequence handles the i-th chunk
// from the one holding token from_len[b] (the last chunk when from_len is
// NULL); nothing happens for a sequence with from_len[b] >= its length.
template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_meta_kernel(KvView kv, ChunkView ch, T *__restrict__ kmin,
                                                         T *__restrict__ kmax, float *__restrict__ cen,
                                                         uint32_t which, const int32_t *__restrict__ from_len,
                                                         int max_touched) {
    constexpr int EPL = 16 / (int)sizeof(T);  // dimensions per 16-byte lane load
    constexpr int NG = D / EPL;                // lanes per token row
    constexpr int TPW = 64 / NG;               // token rows per wave instruction
    const int lane = threadIdx.x & 63, dg = lane % NG, j = lane / NG;
    int c = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int h = blockIdx.y, b = blockIdx.z;
    const int L = kv.seq_lens[b];
    const int32_t *st = ch.starts ? ch.starts + (int64_t)b * (ch.max_chunks + 1) : nullptr;
    const int n = st ? ch.num[b] : (L + kv.page - 1) >> kv.log2page;
    if (max_touched > 0) {
        if (c >= max_touched) return;
        int c0 = n - 1;
        if (from_len) {
            const int f = from_len[b];
            if (f >= L) return;
            if (st) {  // last chunk starting at or before token f
                int lo = 0, hi = n - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (st[mid] <= f) lo = mid; else hi = mid - 1;
                }
                c0 = lo;
            } else {
                c0 = f >> kv.log2page;
            }
        }
        c += c0;
    }
    if (c >= n) return;
    int s, e;
    if (st) {
        s = st[c];
        e = st[c + 1];
    } else {
        s = c << kv.log2page;
        e = min(s + kv.page, L);
    }
    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh + dg * EPL;
    const int64_t bt_row = (int64_t)b * kv.max_pages;
    // fixed pages: the chunk is page c
    const int64_t phys_c = st ? 0 : (kv.bt ? kv.bt[bt_row + c] : bt_row + c);
    float lo[EPL], hi[EPL], sum[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        lo[i] = INFINITY;
        hi[i] = -INFINITY;
        sum[i] = 0.f;
    }
#pragma unroll 4
    for (int t = s + j; t < e; t += TPW) {
        const int page = t >> kv.log2page, slot = t & (kv.page - 1);
        const int64_t phys = st ? (kv.bt ? kv.bt[bt_row + page] : bt_row + page) : phys_c;
        const uint4 w = *reinterpret_cast<const uint4 *>(kb + phys * kv.sp + (int64_t)slot * kv.st);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        float x[EPL];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(T) == 2) {
                x[2 * i] = bf16_lo(ww[i]);
                x[2 * i + 1] = bf16_hi(ww[i]);
            } else {
                x[i] = __uint_as_float(ww[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            lo[i] = fminf(lo[i], x[i]);
            hi[i] = fmaxf(hi[i], x[i]);
            sum[i] += x[i];
        }
    }
    // combine the TPW lanes of each dimension group (lanes dg + NG * j)
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        if constexpr (NG <= 8) {  // lane ^ 8 is lane + 8 mod 16 inside a row
            lo[i] = fminf(lo[i], __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(lo[i]), 0x128, 0xf, 0xf, false)));
            hi[i] = fmaxf(hi[i], __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(hi[i]), 0x128, 0xf, 0xf, false)));
            sum[i] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sum[i]), 0x128, 0xf, 0xf, false));
        }
        if constexpr (NG <= 16) {
            const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(lo[i]), __float_as_int(lo[i]), false, false);
            lo[i] = fminf(__int_as_float(a[0]), __int_as_float(a[1]));
            const auto bb = __builtin_amdgcn_permlane16_swap(__float_as_int(hi[i]), __float_as_int(hi[i]), false, false);
            hi[i] = fmaxf(__int_as_float(bb[0]), __int_as_float(bb[1]));
            const auto cc = __builtin_amdgcn_permlane16_swap(__float_as_int(sum[i]), __float_as_int(sum[i]), false, false);
            sum[i] = __int_as_float(cc[0]) + __int_as_float(cc[1]);
        }
        {
            const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(lo[i]), __float_as_int(lo[i]), false, false);
            lo[i] = fminf(__int_as_float(a[0]), __int_as_float(a[1]));
            const auto bb = __builtin_amdgcn_permlane32_swap(__float_as_int(hi[i]), __float_as_int(hi[i]), false, false);
            hi[i] = fmaxf(__int_as_float(bb[0]), __int_as_float(bb[1]));
            const auto cc = __builtin_amdgcn_permlane32_swap(__float_as_int(sum[i]), __float_as_int(sum[i]), false, false);
            sum[i] = __int_as_float(cc[0]) + __int_as_float(cc[1]);
        }
    }
    if (j != 0) return;
    const int64_t o = (((int64_t)b * kv.hkv + h) * ch.max_chunks + c) * D + dg * EPL;
    if (which & BSA_META_ENVELOPE) {
        if constexpr (sizeof(T) == 2) {
            uint32_t mn[4], mx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mn[i] = uint32_t(f32_to_bf16_exact(lo[2 * i])) | (uint32_t(f32_to_bf16_exact(lo[2 * i + 1])) << 16);
                mx[i] = uint32_t(f32_to_bf16_exact(hi[2 * i])) | (uint32_t(f32_to_bf16_exact(hi[2 * i + 1])) << 16);
            }
            *reinterpret_cast<uint4 *>(kmin + o) = make_uint4(mn[0], mn[1], mn[2], mn[3]);
            *reinterpret_cast<uint4 *>(kmax + o) = make_uint4(mx[0], mx[1], mx[2], mx[3]);
        } else {
            *reinterpret_cast<float4 *>(kmin + o) = make_float4(lo[0], lo[1], lo[2], lo[3]);
            *reinterpret_cast<float4 *>(kmax + o) = make_float4(hi[0], hi[1], hi[2], hi[3]);
        }
    }
    if (which & BSA_META_CENTROID) {
        const float n_tok = float(e - s);
#pragma unroll
        for (int i = 0; i < EPL; i += 4)
            *reinterpret_cast<float4 *>(cen + o + i) =
                make_float4(sum[i] / n_tok, sum[i + 1] / n_tok, sum[i + 2] / n_tok, sum[i + 3] / n_tok);
    }
}

hipError_t launch_chunk_meta(const KvView &kv, const ChunkView &ch, void *kmin, void *kmax, float *cen,
                             uint32_t which, const int32_t *from_len, int32_t max_touched, hipStream_t s) {
    const int span = max_touched > 0 ? max_touched : ch.max_chunks;
    dim3 grid((span + 3) / 4, kv.hkv, kv.batch), block(256);
#define BSA_META(T, D)                                                                                       \
    hipLaunchKernelGGL((chunk_meta_kernel<T, D>), grid, block, 0, s, kv, ch, (T *)kmin, (T *)kmax, cen, which, \
                       from_len, max_touched)
    if (kv.dtype == BSA_BF16) {
        if (kv.d == 128)
            BSA_META(uint16_t, 128);
        else
            BSA_META(uint16_t, 64);
    } else {
        if (kv.d == 128)
            BSA_META(float, 128);
        else
            BSA_META(float, 64);
    }
#undef BSA_META
    return hipGetLastError();
}

}  // namespace bsa
