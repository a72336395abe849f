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
// of K, 1/8 (bf16 envelope) of it written back.
#include "bsa_internal.h"

namespace bsa {

template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_meta_kernel(KvView kv, ChunkView ch, T *__restrict__ kmin,
                                                         T *__restrict__ kmax, float *__restrict__ cen,
                                                         uint32_t which) {
    constexpr int VPL = D / 64;  // dims per lane
    const int lane = threadIdx.x & 63;
    const int c = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int h = blockIdx.y, b = blockIdx.z;
    const int L = kv.seq_lens[b];
    int s, e, n;
    if (ch.starts) {
        n = ch.num[b];
        if (c >= n) return;
        s = ch.starts[(int64_t)b * (ch.max_chunks + 1) + c];
        e = ch.starts[(int64_t)b * (ch.max_chunks + 1) + c + 1];
    } else {
        n = (L + kv.page - 1) >> kv.log2page;
        if (c >= n) return;
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
                             uint32_t which, hipStream_t s) {
    dim3 grid((ch.max_chunks + 3) / 4, kv.hkv, kv.batch), block(256);
    if (kv.dtype == BSA_BF16) {
        if (kv.d == 128)
            hipLaunchKernelGGL((chunk_meta_kernel<uint16_t, 128>), grid, block, 0, s, kv, ch, (uint16_t *)kmin,
                               (uint16_t *)kmax, cen, which);
        else
            hipLaunchKernelGGL((chunk_meta_kernel<uint16_t, 64>), grid, block, 0, s, kv, ch, (uint16_t *)kmin,
                               (uint16_t *)kmax, cen, which);
    } else {
        if (kv.d == 128)
            hipLaunchKernelGGL((chunk_meta_kernel<float, 128>), grid, block, 0, s, kv, ch, (float *)kmin,
                               (float *)kmax, cen, which);
        else
            hipLaunchKernelGGL((chunk_meta_kernel<float, 64>), grid, block, 0, s, kv, ch, (float *)kmin,
                               (float *)kmax, cen, which);
    }
    return hipGetLastError();
}

}  // namespace bsa
