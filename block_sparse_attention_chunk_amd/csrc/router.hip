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
//          are padded with sentinels so every tile has the same dispatch shape;
//          selection and expansion form one code path.
// Readings: sigma per KV head (selection is per KV head); sigma = 0 when the top
// k+1 scores tie; tiles seeing <= k blocks have no cut-off (sigma = 1, never
// triggered, not part of the quantile); quantile by linear interpolation
// between order statistics; strict '<'; sentinel -1 after ascending ids.
//
// Two launches, no sorting:
//  (1) router_select_kernel, one workgroup per (tile, KV head): the radix
//      select of radix_select.h keeps the top max(rho*k, k+1) blocks of the
//      score order, emitted in ascending block order; each kept block counts
//      the kept blocks ranked above it (its rank in the score order), which
//      gives s_(0), s_(k-1), s_(k) for sigma and splits the kept set into the
//      top k (A) and ranks k .. rho*k-1 (B).  The kv_idx row is written as the
//      expansion for both outcomes at once: A ascending, then B ascending,
//      then -1.
//  (2) router_finish_kernel, a few tiles per workgroup: every workgroup forms
//      sigma_bar of all tiles and the quantile itself (a radix select of the
//      order statistics over the eligible tiles; the same arithmetic in every
//      workgroup, so every one finds the same threshold -- the only
//      device-wide dependency of the router), then for its own tiles writes
//      sigma_bar and the trigger flag and finishes the rows: an untriggered
//      tile's row stops after A (sentinels over B), a triggered tile's row
//      merges the two ascending runs in place.
#include "bsa_internal.h"
#include "radix_select.h"

namespace bsa {

constexpr int kMaxList = 256;

__device__ __forceinline__ int tile_visible(int t, int n_blocks, int causal) {
    return causal ? min(t + 1, n_blocks) : n_blocks;
}


// Loads the n visible scores of one row (PER per thread, NT * PER >= n) and
// keeps the top `want` of the score order in kkey / kid, in ascending block
// order; returns the number kept.
template <int NT, int PER>
__device__ __forceinline__ int select_row(const float *__restrict__ row, int n, int want, RadixShared &sh,
                                          uint32_t *kkey, int *kid) {
    const int base = threadIdx.x * PER;
    float raw[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) raw[i] = row[min(base + i, n - 1)];   // visible blocks only
    uint32_t keys[PER];
    int wts[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        keys[i] = base + i < n ? float_key(raw[i]) : 0u;
        wts[i] = 1;
    }
    return radix_select_prefix_emit<NT, PER>(
        keys, wts, base, n, want, true, [](int) {},
        [&](bool keep, int pos, int idx, int i) {
            if (keep && pos < kMaxList) {
                kkey[pos] = keys[i];
                kid[pos] = idx;
            }
        },
        sh);
}

template <int NT, int PER>
__global__ __launch_bounds__(NT) void router_select_kernel(const float *__restrict__ ts, int n_blocks, int hkv,
                                                           int causal, int k, int rho, float *__restrict__ sigma,
                                                           int32_t *__restrict__ kv_idx) {
    __shared__ RadixShared sh;
    __shared__ uint32_t kkey[kMaxList];   // kept blocks in ascending block order: key, id
    __shared__ int kid[kMaxList];
    __shared__ uint32_t rkey[3];          // keys at ranks 0, k-1, k
    args_ready(ts, n_blocks, hkv, causal, k, rho, sigma, kv_idx);
    // KV heads inner and the last tile first: a causal tile's work grows with
    // its index, so the heaviest rows are dispatched first and the lightest
    // fill the tail
    const int h = blockIdx.x, t = gridDim.y - 1 - blockIdx.y;
    const int n = tile_visible(t, n_blocks, causal);
    const int width = rho * k;
    const int want = min(max(width, k + 1), n);
    const float *row = ts + ((int64_t)t * hkv + h) * n_blocks;
    // a causal tile sees only the blocks up to its own, so earlier tiles take
    // a quarter, a half or three quarters of the candidate slots per thread
    // (the choice is uniform over the workgroup)
    constexpr int P1 = PER >= 4 ? PER / 4 : 1, P2 = PER >= 2 ? PER / 2 : 1, P3 = PER >= 4 ? 3 * PER / 4 : PER;
    int cnt;
    if (n <= NT * P1)
        cnt = select_row<NT, P1>(row, n, want, sh, kkey, kid);
    else if (n <= NT * P2)
        cnt = select_row<NT, P2>(row, n, want, sh, kkey, kid);
    else if (n <= NT * P3)
        cnt = select_row<NT, P3>(row, n, want, sh, kkey, kid);
    else
        cnt = select_row<NT, PER>(row, n, want, sh, kkey, kid);
    __syncthreads();
    // rank of kept block p in the score order (descending key, lower block
    // first): kept blocks sit in ascending block order, so an equal key ranks
    // above p exactly when it sits before p
    const int p = threadIdx.x;
    int r = 0;
    uint32_t kp = 0;
    if (p < cnt) {
        kp = kkey[p];
        for (int q0 = 0; q0 < cnt; q0 += 16) {   // 16 reads in flight, then 16 compares
            uint32_t kq[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) kq[j] = kkey[min(q0 + j, kMaxList - 1)];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int q = q0 + j;
                r += (q < cnt && (kq[j] > kp || (kq[j] == kp && q < p))) ? 1 : 0;
            }
        }
        if (r == 0) rkey[0] = kp;
        if (r == k - 1) rkey[1] = kp;
        if (r == k) rkey[2] = kp;
    }
    // positions: A = ranks < k, ascending; B = ranks k .. width-1, ascending
    const bool in_a = p < cnt && r < k, in_b = p < cnt && r >= k && r < width;
    int a = in_a ? 1 : 0, b = in_b ? 1 : 0, ta, tb;
    block_scan_pair<NT>(a, b, sh, ta, tb);   // inclusive; totals |A|, |B|
    int32_t *dst = kv_idx + ((int64_t)t * hkv + h) * width;
    if (in_a) dst[a - 1] = kid[p];
    if (in_b) dst[ta + b - 1] = kid[p];
    for (int i = ta + tb + (int)threadIdx.x; i < width; i += NT) dst[i] = -1;
    __syncthreads();   // rkey written
    if (threadIdx.x == 0) {
        double sg = 1.0;
        if (n > k) {
            const double s0 = key_float(rkey[0]), sk1 = key_float(rkey[1]), sk = key_float(rkey[2]);
            sg = (s0 == sk) ? 0.0 : (sk1 - sk) / (s0 - sk);
        }
        sigma[(int64_t)t * hkv + h] = (float)sg;
    }
}

// sigma_bar of tile t: the mean over KV heads in double (heads added in
// order), stored as float.  HK > 0: the head count known at compile time, so
// every load of a thread's candidates is in flight at once.
template <int HK>
__device__ __forceinline__ float sigma_mean(const float *__restrict__ sigma, int t, int hkv) {
    double acc = 0.0;
    if constexpr (HK > 0) {
        float x[HK];
#pragma unroll
        for (int h = 0; h < HK; ++h) x[h] = sigma[(int64_t)t * HK + h];
#pragma unroll
        for (int h = 0; h < HK; ++h) acc += (double)x[h];
        return (float)(acc / HK);
    } else {
        for (int h = 0; h < hkv; ++h) acc += (double)sigma[(int64_t)t * hkv + h];
        return (float)(acc / hkv);
    }
}

constexpr int kFinThreads = 512;
constexpr int kFinWaves = kFinThreads / 64;
constexpr int kFinPer = 16;        // quantile candidates per thread: up to 8192 tiles
constexpr int kFinRows = 32;       // (tile, KV head) rows finished per workgroup and round

// Tiles per finishing workgroup: up to kFinRows rows (at least one tile).
__host__ __device__ __forceinline__ int fin_tiles(int hkv) { return hkv >= kFinRows ? 1 : kFinRows / hkv; }

// Order statistics lo and lo + 1 (ascending) of the eligible tiles'
// sigma_bar, tiles [e0, e0 + m): a radix select keeps the lo + 1 smallest
// (keys inverted); x_lo is the largest kept value and x_hi the smallest value
// not kept.  FPER candidates per thread, kFinThreads * FPER >= m.
template <int HK, int FPER>
__device__ __forceinline__ void quantile_pair(const float *__restrict__ sigma, int e0, int m, int lo, int hkv,
                                              RadixShared &sh, float (&red)[2][kFinWaves], float &x_lo,
                                              float &x_hi) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int base = threadIdx.x * FPER;
    float v[FPER];
    uint32_t keys[FPER];
    int wts[FPER];
#pragma unroll
    for (int i = 0; i < FPER; ++i) {
        const int c = base + i;
        v[i] = c < m ? sigma_mean<HK>(sigma, e0 + c, hkv) : 0.f;
        keys[i] = c < m ? ~float_key(v[i]) : 0u;
        wts[i] = 1;
    }
    float kept_max = -INFINITY, rest_min = INFINITY;
    radix_select_prefix_emit<kFinThreads, FPER>(
        keys, wts, base, m, lo + 1, true, [](int) {},
        [&](bool keep, int, int idx, int i) {
            if (idx < m) {
                kept_max = keep ? fmaxf(kept_max, v[i]) : kept_max;
                rest_min = keep ? rest_min : fminf(rest_min, v[i]);
            }
        },
        sh);
    kept_max = wave_max_all(kept_max);
    rest_min = -wave_max_all(-rest_min);
    if (lane == 0) {
        red[0][w] = kept_max;
        red[1][w] = rest_min;
    }
    __syncthreads();
    x_lo = -INFINITY;
    x_hi = INFINITY;
#pragma unroll
    for (int i = 0; i < kFinWaves; ++i) {
        x_lo = fmaxf(x_lo, red[0][i]);
        x_hi = fminf(x_hi, red[1][i]);
    }
}

template <int HK>
__global__ __launch_bounds__(kFinThreads) void router_finish_kernel(const float *__restrict__ sigma, int n_tiles,
                                                                    int hkv, int n_blocks, int causal, int k,
                                                                    int rho, float quantile, float fixed,
                                                                    float *__restrict__ sigma_bar,
                                                                    uint8_t *__restrict__ triggered,
                                                                    float *__restrict__ threshold,
                                                                    int32_t *__restrict__ kv_idx) {
    __shared__ RadixShared sh;
    __shared__ float red[2][kFinWaves];
    __shared__ int32_t rowbuf[kFinRows][kMaxList];
    __shared__ float sb_s[kFinRows];
    args_ready(sigma, n_tiles, hkv, n_blocks, causal, k, rho, quantile, fixed, kv_idx);
    const int width = rho * k;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tpw = fin_tiles(hkv);
    const int t0 = blockIdx.x * tpw;
    const int nt_w = min(tpw, n_tiles - t0);
    const int rows = nt_w * hkv;
    // eligible tiles form the range [e0, n_tiles): causal tile t sees
    // min(t + 1, n_blocks) blocks, so it has a cut-off exactly when t >= k
    // (and n_blocks > k); every tile sees n_blocks blocks otherwise
    const int e0 = n_blocks > k ? (causal ? min(k, n_tiles) : 0) : n_tiles;
    const int m = n_tiles - e0;

    // the first round of this workgroup's rows is requested before the
    // threshold is known (it does not depend on it), and so is sigma_bar of
    // its tiles
    auto load_rows = [&](int r0) {
        for (int rr = w; rr < min(kFinRows, rows - r0); rr += kFinWaves) {
            const int t = t0 + (r0 + rr) / hkv, h = (r0 + rr) - ((r0 + rr) / hkv) * hkv;
            const int32_t *row = kv_idx + ((int64_t)t * hkv + h) * width;
            for (int i = lane; i < width; i += 64) rowbuf[rr][i] = row[i];
        }
    };
    load_rows(0);
    if ((int)threadIdx.x < nt_w) sb_s[threadIdx.x] = sigma_mean<HK>(sigma, t0 + threadIdx.x, hkv);

    double tau;
    if (!isnan(fixed)) {
        tau = fixed;
    } else if (m == 0) {
        tau = NAN;
    } else {
        const double pos = (double)(m - 1) * (double)quantile;
        const int lo = (int)floor(pos);
        const double frac = pos - lo;
        float x_lo, x_hi;
        if (m <= kFinThreads * 4)
            quantile_pair<HK, 4>(sigma, e0, m, lo, hkv, sh, red, x_lo, x_hi);
        else if (m <= kFinThreads * 8)
            quantile_pair<HK, 8>(sigma, e0, m, lo, hkv, sh, red, x_lo, x_hi);
        else
            quantile_pair<HK, kFinPer>(sigma, e0, m, lo, hkv, sh, red, x_lo, x_hi);
        tau = lo + 1 < m ? (double)x_lo + frac * ((double)x_hi - (double)x_lo) : (double)x_lo;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) threshold[0] = (float)tau;
    __syncthreads();   // sb_s and the first round of rows are in LDS
    if ((int)threadIdx.x < nt_w) {
        const int t = t0 + threadIdx.x;
        const float sb = sb_s[threadIdx.x];
        sigma_bar[t] = sb;
        triggered[t] = (t >= e0 && (double)sb < tau) ? 1 : 0;
    }

    // finish the rows, one wave per (tile, KV head) row
    for (int r0 = 0; r0 < rows; r0 += kFinRows) {
        if (r0 > 0) {
            __syncthreads();   // every wave is done with the previous round
            load_rows(r0);
            __syncthreads();
        }
        for (int rr = w; rr < min(kFinRows, rows - r0); rr += kFinWaves) {
            const int tl = (r0 + rr) / hkv, h = (r0 + rr) - tl * hkv, t = t0 + tl;
            const int n = tile_visible(t, n_blocks, causal);
            const int na = min(k, n), nb = min(width, n) - na;   // |A|, |B|
            const bool trig = t >= e0 && (double)sb_s[tl] < tau;
            int32_t *row = kv_idx + ((int64_t)t * hkv + h) * width;
            if (!trig) {
                for (int i = na + lane; i < na + nb; i += 64) row[i] = -1;
                continue;
            }
            // merge A = row[0, na) and B = row[na, na + nb), both ascending and
            // disjoint: an element's place is its index in its own run plus
            // the number of smaller elements in the other run
            const int32_t *buf = rowbuf[rr];
            for (int i = lane; i < na + nb; i += 64) {
                const int x = buf[i];
                const bool from_a = i < na;
                int lo2 = from_a ? na : 0, hi2 = from_a ? na + nb : na;   // search the other run
                const int start = lo2;
                while (lo2 < hi2) {
                    const int mid = (lo2 + hi2) >> 1;
                    if (buf[mid] < x) lo2 = mid + 1;
                    else hi2 = mid;
                }
                row[(from_a ? i : i - na) + (lo2 - start)] = x;
            }
        }
    }
}

hipError_t launch_router(const float *ts, int32_t n_tiles, int32_t hkv, int32_t n_blocks, int32_t causal, int32_t k,
                         int32_t rho, float quantile, float fixed, int32_t *kv_idx, float *sigma, float *sigma_bar,
                         uint8_t *triggered, float *threshold, void *, hipStream_t s) {
    dim3 grid(hkv, n_tiles);
    // the kept list (<= 256 blocks) needs one thread per kept block (measured
    // at 131,072 tokens: 128 threads x 16 candidates 58 us for the router,
    // one wave x 32 candidates 70 us)
    const int want = max(rho * k, k + 1);
    if (n_blocks <= 128 * 16 && want <= 128)
        hipLaunchKernelGGL((router_select_kernel<128, 16>), grid, dim3(128), 0, s, ts, n_blocks, hkv, causal, k, rho,
                           sigma, kv_idx);
    else if (n_blocks <= 256 * 16)
        hipLaunchKernelGGL((router_select_kernel<256, 16>), grid, dim3(256), 0, s, ts, n_blocks, hkv, causal, k, rho,
                           sigma, kv_idx);
    else
        hipLaunchKernelGGL((router_select_kernel<1024, 8>), grid, dim3(1024), 0, s, ts, n_blocks, hkv, causal, k, rho,
                           sigma, kv_idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tpw = fin_tiles(hkv);
    const dim3 fg((n_tiles + tpw - 1) / tpw), fb(kFinThreads);
#define BSA_FIN(HK)                                                                                                \
    hipLaunchKernelGGL(router_finish_kernel<HK>, fg, fb, 0, s, sigma, n_tiles, hkv, n_blocks, causal, k, rho, quantile, \
                       fixed, sigma_bar, triggered, threshold, kv_idx)
    switch (hkv) {
    case 1: BSA_FIN(1); break;
    case 2: BSA_FIN(2); break;
    case 4: BSA_FIN(4); break;
    case 8: BSA_FIN(8); break;
    default: BSA_FIN(0); break;
    }
#undef BSA_FIN
    return hipGetLastError();
}

}  // namespace bsa
