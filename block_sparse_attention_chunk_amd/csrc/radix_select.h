// radix_select.h -- weighted radix select of a score-order prefix, shared by
// the decode selection and the router (one 256-thread workgroup per row).
#pragma once

#include "bsa_internal.h"

namespace bsa {

constexpr int kSelThreads = 256;

// Weighted radix select of the longest (score desc, index asc) prefix of keys[0..n)
// with total weight <= budget.  Writes the kept indices ascending to dst (at most
// dst_cap of them) and returns the count.  Must be called by all 256 threads.
template <typename WeightFn>
__device__ __forceinline__ int radix_select_prefix(const uint32_t *keys, int n, int64_t budget, WeightFn weight,
                                                   int *dst, int dst_cap, int *hist, int *scan, int *bcast) {
    const int tid = threadIdx.x;
    // total weight
    int64_t local = 0;
    for (int i = tid; i < n; i += kSelThreads) local += weight(i);
    int tot;
    (void)block_scan_incl_256((int)local, scan, &tot);
    const bool all = (int64_t)tot <= budget;
    uint32_t T = 0;
    int remaining = 0;
    if (!all) {
        uint32_t prefix = 0, pmask = 0;
        int wabove = 0;
        const int bud = (int)budget;  // < tot, fits in int
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            hist[tid] = 0;
            __syncthreads();
            for (int i = tid; i < n; i += kSelThreads) {
                const uint32_t k = keys[i];
                if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], weight(i));
            }
            __syncthreads();
            const int v = hist[255 - tid];
            int dummy;
            const int incl = block_scan_incl_256(v, scan, &dummy);
            if (wabove + incl > bud && wabove + incl - v <= bud) {
                bcast[0] = 255 - tid;
                bcast[1] = wabove + incl - v;
            }
            __syncthreads();
            prefix |= uint32_t(bcast[0]) << shift;
            pmask |= 255u << shift;
            wabove = bcast[1];
            __syncthreads();
        }
        T = prefix;
        remaining = bud - wabove;
    }
    // ordered compaction
    int carry_eq = 0, out_pos = 0;
    for (int base = 0; base < n; base += kSelThreads) {
        const int i = base + tid;
        const bool valid = i < n;
        const uint32_t k = valid ? keys[i] : 0u;
        const int w = valid ? weight(i) : 0;
        const bool is_eq = valid && !all && k == T;
        int teq;
        const int incl_eq = block_scan_incl_256(is_eq ? w : 0, scan, &teq) + carry_eq;
        const bool sel = valid && (all || k > T || (is_eq && incl_eq <= remaining));
        int tsel;
        const int pos = block_scan_incl_256(sel ? 1 : 0, scan, &tsel) - (sel ? 1 : 0) + out_pos;
        if (sel && pos < dst_cap) dst[pos] = i;
        carry_eq += teq;
        out_pos += tsel;
    }
    __syncthreads();  // dst may be LDS read by other threads after the call
    return min(out_pos, dst_cap);
}

}  // namespace bsa
