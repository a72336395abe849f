// router.hip -- the uncertainty router over query tiles.
//
// Source: "Technische Samenvatting: Onzekerheidsgestuurde Selectie voor
// Blok-schaarse Aandacht", section "Methodologie":
//  step 2  per-tile top-k over the tile's block scores gives kv_idx;
//  step 3  cut-off margin sigma = (s_(k-1) - s_(k)) / (s_(0) - s_(k)) over the
//          descending block scores (sigma near 1: decisive; near 0: the k-th
//          and (k+1)-th blocks tie);
//  step 4  sigma averaged over heads into one value per tile, triggered when it
//          falls below a per-layer empirical quantile;
//  step 5  triggered tiles attend to the top rho*k blocks, the others keep k and
//          are padded with sentinels so every tile has the same dispatch shape.
// Readings: sigma per KV head (selection is per KV head); sigma = 0 when the top
// k+1 scores tie; tiles seeing <= k blocks have no cut-off (sigma = 1, never
// triggered, not part of the quantile); quantile by linear interpolation
// between order statistics; strict '<'; sentinel -1 after ascending ids.
//
// Three launches: (1) one workgroup per (tile, KV head) selects the top
// max(rho*k, k+1) blocks with the radix select of radix_select.h, sorts them (bitonic in LDS) and writes sigma plus the score-ordered
// list; (2) one workgroup computes sigma_bar, the threshold and the trigger
// flags (the path's only device-wide dependency); (3) one workgroup per
// (tile, KV head) emits the ascending, sentinel-padded kv_idx row.
#include "bsa_internal.h"
#include "radix_select.h"

namespace bsa {

constexpr int kRtThreads = 256;
constexpr int kMaxList = 256;

__device__ __forceinline__ int tile_visible(int t, int n_blocks, int causal) {
    return causal ? min(t + 1, n_blocks) : n_blocks;
}

// Bitonic sort of n2 (power of two, <= 256) 64-bit values in LDS, descending.
__device__ void bitonic_desc_u64(uint64_t *v, int n2) {
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const int i = threadIdx.x;
            if (i < n2) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool desc = (i & size) == 0;
                    const uint64_t a = v[i], c = v[j];
                    if (desc ? (a < c) : (a > c)) {
                        v[i] = c;
                        v[j] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
}

constexpr int kRtPer = 8;   // candidates per thread: up to 8 * NT blocks per tile

template <int NT>
__global__ __launch_bounds__(NT) void router_topk_kernel(const float *__restrict__ ts, int n_blocks, int hkv,
                                                            int causal, int k, int rho, float *__restrict__ sigma,
                                                            int32_t *__restrict__ top) {
    __shared__ RadixShared sh;
    __shared__ uint32_t skeys[NT * kRtPer];
    __shared__ int sel[kMaxList];
    __shared__ uint64_t list[kMaxList];
    const int t = blockIdx.x, h = blockIdx.y;
    const int n = tile_visible(t, n_blocks, causal);
    const int width = rho * k;
    const int want = min(max(width, k + 1), n);
    const float *row = ts + ((int64_t)t * hkv + h) * n_blocks;
    const int base = threadIdx.x * kRtPer;
    uint32_t keys[kRtPer];
    int wts[kRtPer];
#pragma unroll
    for (int i = 0; i < kRtPer; ++i) {
        keys[i] = base + i < n ? float_key(row[base + i]) : 0u;
        wts[i] = 1;
        if (base + i < n) skeys[base + i] = keys[i];
    }
    const int cnt = radix_select_prefix<NT, kRtPer>(keys, wts, base, n, want, true, sel, kMaxList, sh);
    __syncthreads();
    int n2 = 1;
    while (n2 < cnt) n2 <<= 1;
    for (int i = threadIdx.x; i < n2; i += NT)
        list[i] = i < cnt ? ((uint64_t)skeys[sel[i]] << 32) | (uint64_t)(0xffffffffu - (uint32_t)sel[i]) : 0ull;
    __syncthreads();
    bitonic_desc_u64(list, n2);
    int32_t *dst = top + ((int64_t)t * hkv + h) * width;
    for (int i = threadIdx.x; i < width; i += NT)
        dst[i] = i < min(cnt, width) ? (int32_t)(0xffffffffu - (uint32_t)(list[i] & 0xffffffffu)) : -1;
    if (threadIdx.x == 0) {
        double sg = 1.0;
        if (n > k) {
            const double s0 = key_float((uint32_t)(list[0] >> 32));
            const double sk1 = key_float((uint32_t)(list[k - 1] >> 32));
            const double sk = key_float((uint32_t)(list[k] >> 32));
            sg = (s0 == sk) ? 0.0 : (sk1 - sk) / (s0 - sk);
        }
        sigma[(int64_t)t * hkv + h] = (float)sg;
    }
}

// One workgroup: sigma_bar, the quantile threshold over eligible tiles, trigger flags.
constexpr int kQThreads = 1024;

__global__ __launch_bounds__(kQThreads) void router_threshold_kernel(const float *__restrict__ sigma, int n_tiles,
                                                                     int hkv, int n_blocks, int causal, int k,
                                                                     float quantile, float fixed,
                                                                     float *__restrict__ sigma_bar,
                                                                     uint8_t *__restrict__ triggered,
                                                                     float *__restrict__ threshold) {
    extern __shared__ float vals[];   // next power of two >= n_tiles
    __shared__ int cnt_s;
    __shared__ double tau_s;
    if (threadIdx.x == 0) cnt_s = 0;
    __syncthreads();
    auto mean_sigma = [&](int t) {
        double acc = 0.0;
        for (int h = 0; h < hkv; ++h) acc += (double)sigma[(int64_t)t * hkv + h];
        return (float)(acc / hkv);
    };
    int n2 = 1;
    while (n2 < n_tiles) n2 <<= 1;
    // eligible values first (order irrelevant: they are sorted next), +inf padding
    for (int t = threadIdx.x; t < n2; t += kQThreads) vals[t] = INFINITY;
    __syncthreads();
    for (int t = threadIdx.x; t < n_tiles; t += kQThreads) {
        const float sb = mean_sigma(t);
        sigma_bar[t] = sb;
        if (tile_visible(t, n_blocks, causal) > k) {
            const int slot = atomicAdd(&cnt_s, 1);
            vals[slot] = sb;
        }
    }
    __syncthreads();
    const int m = cnt_s;
    // ascending bitonic sort of n2 floats
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < n2; i += kQThreads) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool asc = (i & size) == 0;
                    const float a = vals[i], c = vals[j];
                    if (asc ? (a > c) : (a < c)) {
                        vals[i] = c;
                        vals[j] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    if (threadIdx.x == 0) {
        double tau;
        if (!isnan(fixed)) {
            tau = fixed;
        } else if (m == 0) {
            tau = NAN;
        } else {
            const double pos = (double)(m - 1) * (double)quantile;
            const int lo = (int)floor(pos);
            const double frac = pos - lo;
            tau = lo + 1 < m ? (double)vals[lo] + frac * ((double)vals[lo + 1] - (double)vals[lo]) : (double)vals[lo];
        }
        tau_s = tau;
        threshold[0] = (float)tau;
    }
    __syncthreads();
    const double tau = tau_s;
    for (int t = threadIdx.x; t < n_tiles; t += kQThreads) {
        const bool elig = tile_visible(t, n_blocks, causal) > k;
        triggered[t] = (elig && (double)mean_sigma(t) < tau) ? 1 : 0;
    }
}

__global__ __launch_bounds__(kRtThreads) void router_emit_kernel(const int32_t *__restrict__ top,
                                                                 const uint8_t *__restrict__ triggered, int n_blocks,
                                                                 int hkv, int causal, int k, int rho,
                                                                 int32_t *__restrict__ kv_idx) {
    __shared__ uint32_t v[kMaxList];
    const int t = blockIdx.x, h = blockIdx.y;
    const int width = rho * k;
    const int n = tile_visible(t, n_blocks, causal);
    const int keep = min(triggered[t] ? width : k, n);
    int n2 = 1;
    while (n2 < keep) n2 <<= 1;
    const int32_t *src = top + ((int64_t)t * hkv + h) * width;
    for (int i = threadIdx.x; i < n2; i += kRtThreads) v[i] = i < keep ? (uint32_t)src[i] : 0xffffffffu;
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const int i = threadIdx.x;
            if (i < n2) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool asc = (i & size) == 0;
                    const uint32_t a = v[i], c = v[j];
                    if (asc ? (a > c) : (a < c)) {
                        v[i] = c;
                        v[j] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    int32_t *dst = kv_idx + ((int64_t)t * hkv + h) * width;
    for (int i = threadIdx.x; i < width; i += kRtThreads) dst[i] = i < keep ? (int32_t)v[i] : -1;
}

hipError_t launch_router(const float *ts, int32_t n_tiles, int32_t hkv, int32_t n_blocks, int32_t causal, int32_t k,
                         int32_t rho, float quantile, float fixed, int32_t *kv_idx, float *sigma, float *sigma_bar,
                         uint8_t *triggered, float *threshold, void *ws, hipStream_t s) {
    int32_t *top = (int32_t *)ws;
    dim3 grid(n_tiles, hkv);
    if (n_blocks <= 256 * kRtPer)
        hipLaunchKernelGGL(router_topk_kernel<256>, grid, dim3(256), 0, s, ts, n_blocks, hkv, causal, k, rho, sigma,
                           top);
    else
        hipLaunchKernelGGL(router_topk_kernel<1024>, grid, dim3(1024), 0, s, ts, n_blocks, hkv, causal, k, rho, sigma,
                           top);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int n2 = 1;
    while (n2 < n_tiles) n2 <<= 1;
    hipLaunchKernelGGL(router_threshold_kernel, dim3(1), dim3(kQThreads), (size_t)n2 * sizeof(float), s, sigma,
                       n_tiles, hkv, n_blocks, causal, k, quantile, fixed, sigma_bar, triggered, threshold);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(router_emit_kernel, grid, dim3(kRtThreads), 0, s, top, triggered, n_blocks, hkv, causal, k, rho,
                       kv_idx);
    return hipGetLastError();
}

}  // namespace bsa
