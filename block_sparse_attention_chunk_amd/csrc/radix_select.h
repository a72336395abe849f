// radix_select.h -- weighted radix select of a score-order prefix, shared by
// the decode selection and the router.
//
// Candidates are ordered by (score descending, index ascending).  With a
// weight per candidate, the selection is the longest prefix of that order
// whose total weight fits the budget.  Four 8-bit passes over
// order-preserving float keys find the key T of the first candidate that does
// not fit; every key > T is kept, and the candidates with key == T are kept in
// ascending index order while their running weight still fits.  The kept ids
// come out in ascending index order from a block scan, so ties need no sort.
//
// One workgroup of NT threads per row; each thread holds PER consecutive
// candidates in registers (n <= NT * PER).
#pragma once

#include "bsa_internal.h"

namespace bsa {

struct RadixShared {
    int hist[256];
    int wsum[32];       // per-wave partial sums of the block scans
    int digit, wabove;
    long long total;
};

// Inclusive block scan of v over NT threads; *total receives the block sum.
template <int NT>
__device__ __forceinline__ int block_scan_incl(int v, RadixShared &sh, int *total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh.wsum[wid] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int s = sh.wsum[w];
        off += (w < wid) ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return x + off;
}

// keys[PER] / wts[PER]: this thread's candidates (index base + i, valid when
// base + i < n).  Returns the number kept; writes the kept indices ascending to
// dst[0 .. min(count, dst_cap)).
template <int NT, int PER>
__device__ __forceinline__ int radix_select_prefix(const uint32_t (&keys)[PER], const int (&wts)[PER], int base,
                                                   int n, int64_t budget, int *dst, int dst_cap, RadixShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63;
    int my_w = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) my_w += (base + i < n) ? wts[i] : 0;
    int tot;
    (void)block_scan_incl<NT>(my_w, sh, &tot);
    const bool all = (int64_t)tot <= budget;
    uint32_t T = 0;
    int remaining = 0;
    if (!all) {
        uint32_t prefix = 0, pmask = 0;
        int wabove = 0;
        const int bud = (int)budget;  // < tot
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int i = tid; i < 256; i += NT) sh.hist[i] = 0;
            __syncthreads();
            // consecutive candidates mostly share a digit (scores of neighbouring
            // chunks have similar magnitude): add runs of equal digits at once
            int run_d = -1, run_w = 0;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                if (base + i < n && (keys[i] & pmask) == prefix) {
                    const int d = (keys[i] >> shift) & 255u;
                    if (d != run_d) {
                        if (run_w) atomicAdd(&sh.hist[run_d], run_w);
                        run_d = d;
                        run_w = 0;
                    }
                    run_w += wts[i];
                }
            }
            if (run_w) atomicAdd(&sh.hist[run_d], run_w);
            __syncthreads();
            if (tid < 64) {
                // lane L holds digits 255-4L .. 252-4L (descending)
                int h[4], s = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    h[j] = sh.hist[255 - 4 * lane - j];
                    s += h[j];
                }
                int x = s;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(x, o, 64);
                    if (lane >= o) x += y;
                }
                int before = wabove + x - s;  // weight of all higher digits
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (before <= bud && before + h[j] > bud) {
                        sh.digit = 255 - 4 * lane - j;
                        sh.wabove = before;
                    }
                    before += h[j];
                }
            }
            __syncthreads();
            prefix |= uint32_t(sh.digit) << shift;
            pmask |= 255u << shift;
            wabove = sh.wabove;
        }
        T = prefix;
        remaining = bud - wabove;
    }
    // weight of this thread's key == T candidates, then their running prefix
    int eqw = 0;
    if (!all) {
#pragma unroll
        for (int i = 0; i < PER; ++i) eqw += (base + i < n && keys[i] == T) ? wts[i] : 0;
    }
    int teq;
    int run = block_scan_incl<NT>(eqw, sh, &teq) - eqw;  // exclusive
    bool sel[PER];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool valid = base + i < n;
        bool s = valid && (all || keys[i] > T);
        if (valid && !all && keys[i] == T) {
            run += wts[i];
            s = run <= remaining;
        }
        sel[i] = s;
        cnt += s ? 1 : 0;
    }
    int total;
    int pos = block_scan_incl<NT>(cnt, sh, &total) - cnt;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (sel[i]) {
            if (pos < dst_cap) dst[pos] = base + i;
            ++pos;
        }
    }
    (void)lane;
    return min(total, dst_cap);
}

}  // namespace bsa
