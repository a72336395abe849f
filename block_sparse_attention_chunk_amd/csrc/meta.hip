// meta.hip -- per-chunk key metadata (min / max envelope and centroid).
//
// Source: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (method table: envelope = per-dimension min/max of
// a chunk's keys, centroid = mean of a chunk's keys); "Technische Samenvatting
// ... Blok-schaarse Aandacht", section "Methodologie" step 1.
//
// One wave per (sequence, KV head, chunk).  Lanes own consecutive dimensions,
// so every token row is one coalesced 128/256-byte read; the wave walks the
// chunk's tokens in order (the page of each token comes from the block table,
// so variable chunks may cross pages).  min / max are exact, the centroid is a
// float32 sum in token order divided by the token count.  HBM-bound: one read
// of K, 1/8 (bf16 envelope) of it written back.  The same kernel refreshes
// only the chunks that newly appended tokens touched (update mode), with
// results identical to a full rebuild of those chunks.
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
    constexpr int VPL = D / 64;  // dims per lane
    const int lane = threadIdx.x & 63;
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
    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh + lane * VPL;
    float lo[VPL], hi[VPL], sum[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        lo[i] = INFINITY;
        hi[i] = -INFINITY;
        sum[i] = 0.f;
    }
#pragma unroll 4
    for (int t = s; t < e; ++t) {
        const int page = t >> kv.log2page, slot = t & (kv.page - 1);
        const int64_t phys = kv.bt ? kv.bt[(int64_t)b * kv.max_pages + page] : (int64_t)b * kv.max_pages + page;
        const T *row = kb + phys * kv.sp + (int64_t)slot * kv.st;
        float x[VPL];
        if constexpr (sizeof(T) == 2) {
            if constexpr (VPL == 2) {
                uint32_t w = *reinterpret_cast<const uint32_t *>(row);
                x[0] = bf16_lo(w);
                x[1] = bf16_hi(w);
            } else {
                x[0] = bf16_to_f32(*reinterpret_cast<const uint16_t *>(row));
            }
        } else {
#pragma unroll
            for (int i = 0; i < VPL; ++i) x[i] = reinterpret_cast<const float *>(row)[i];
        }
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            lo[i] = fminf(lo[i], x[i]);
            hi[i] = fmaxf(hi[i], x[i]);
            sum[i] += x[i];
        }
    }
    const int64_t o = (((int64_t)b * kv.hkv + h) * ch.max_chunks + c) * D + lane * VPL;
    if (which & BSA_META_ENVELOPE) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            if constexpr (sizeof(T) == 2) {
                reinterpret_cast<uint16_t *>(kmin)[o + i] = f32_to_bf16_exact(lo[i]);
                reinterpret_cast<uint16_t *>(kmax)[o + i] = f32_to_bf16_exact(hi[i]);
            } else {
                kmin[o + i] = lo[i];
                kmax[o + i] = hi[i];
            }
        }
    }
    if (which & BSA_META_CENTROID) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) cen[o + i] = sum[i] / float(e - s);
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
