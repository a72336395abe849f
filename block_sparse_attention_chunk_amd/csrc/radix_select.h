// radix_select.h -- weighted radix select of a score-order prefix, shared by
// the decode selection, the fused selection + decode kernel and the router.
//
// Candidates are ordered by (score descending, index ascending).  With a
// weight per candidate, the selection is the longest prefix of that order
// whose total weight fits the budget.  Up to four 8-bit passes over
// order-preserving float keys find the key T of the first candidate that does
// not fit; every key > T is kept, and the candidates with key == T are kept in
// ascending index order while their running weight still fits.  The kept ids
// come out in ascending index order from one block scan, so ties need no sort.
//
// One workgroup of NT threads per row; each thread holds PER consecutive
// candidates in registers (n <= NT * PER).  The passes start below the leading
// bits that the smallest and the largest key share (scores of one row usually
// share sign and most of the exponent, so a pass over those bits would rank
// nothing).  Per pass: histogram atomics into one of three rotating LDS
// histograms (two sub-histograms, even / odd waves), one barrier, then every
// wave finds the crossing digit itself (lane l owns digits 255-4l .. 252-4l,
// a DPP wave scan gives the weight above them), so no second barrier
// broadcasts it.  A histogram is cleared two passes after it was read, so
// clearing needs no barrier of its own.  The total weight falls out of the
// first pass, and the passes stop early when the cut lands on a digit
// boundary.
#pragma once

#include "bsa_internal.h"

namespace bsa {

struct RadixShared {
    int hist[3][2][256];
    int wsum[2][16];    // per-wave partials of the block scan (<= 16 waves)
    int wext[16];       // per-wave weight of the forced candidates
    int esel;           // number of kept candidates with key == T (-1: all of them)
};

// Inclusive scan over the 64 lanes of a wave with DPP: shifts 1, 2, 4, 8 inside
// each row of 16 (lanes before the row start add 0), then the last lane of
// each row into the next row (rows 1, 3) and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_scan_incl(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Maximum over the 64 lanes of a wave (same shift pattern as the scan; lanes
// outside a shift's source range contribute 0).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Inclusive block scan of two values at once over NT threads; totals in ta /
// tb.  Single use per kernel phase: the per-wave partials are not protected
// against a second scan that starts before every wave has read them.
template <int NT>
__device__ __forceinline__ void block_scan_pair(int &a, int &b, RadixShared &sh, int &ta, int &tb) {
    constexpr int NW = NT / 64;
    static_assert(NW <= 16, "at most 16 waves");
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    a = wave_scan_incl(a);
    b = wave_scan_incl(b);
    if (lane == 63) {
        sh.wsum[0][wid] = a;
        sh.wsum[1][wid] = b;
    }
    __syncthreads();
    int oa = 0, ob = 0;
    ta = 0, tb = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int x = sh.wsum[0][w], y = sh.wsum[1][w];
        oa += (w < wid) ? x : 0;
        ob += (w < wid) ? y : 0;
        ta += x;
        tb += y;
    }
    a += oa;
    b += ob;
}

// keys[PER] / wts[PER] (weights >= 1): this thread's candidates (index
// base + i, valid when base + i < n <= 65535).  Returns the number kept.
// emit(keep, pos, index, i) is called once for every slot i of this thread,
// in order; for a kept candidate, pos is its rank in ascending index order.  A
// thread's kept candidates take consecutive ranks: begin(p) is called once per
// thread, before its first emit, with the rank its first kept candidate gets
// (or would get).  The total weight must stay below 2^31.  `unit` (uniform):
// every weight is 1, so the number of ties kept at the cut follows from the
// counts alone, without a search and its barrier.
template <int NT, int PER, typename Begin, typename Emit>
__device__ __forceinline__ int radix_select_prefix_emit(const uint32_t (&keys)[PER], const int (&wts)[PER], int base,
                                                        int n, int64_t budget, bool unit, Begin begin, Emit emit,
                                                        RadixShared &sh) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, sub = wid & 1;
    const int bud = (int)min(budget, (int64_t)0x7fffffff);
    // Forced candidates (key 0xffffffff, which no finite score has) are kept
    // outright; the passes rank the others.  Their keys all lie between the
    // smallest and the largest of them and so share those two keys' leading
    // bits: the first pass starts below those bits.
    bool cand[PER];
    uint32_t tmax = 0, tnmin = 0;
    int tforced = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool v = base + i < n, f = keys[i] == 0xffffffffu;
        cand[i] = v && !f;
        tmax = max(tmax, cand[i] ? keys[i] : 0u);
        tnmin = max(tnmin, cand[i] ? ~keys[i] : 0u);
        tforced += (v && f) ? wts[i] : 0;
    }
    tmax = wave_max_u32(tmax);
    tnmin = wave_max_u32(tnmin);
    tforced = __builtin_amdgcn_readlane(wave_scan_incl(tforced), 63);
    if (lane == 0) {
        sh.wsum[0][wid] = (int)tmax;
        sh.wsum[1][wid] = (int)tnmin;
        sh.wext[wid] = tforced;
    }
    int *flat0 = &sh.hist[0][0][0];
    for (int i = tid; i < 512; i += NT) flat0[i] = 0;
    if (tid == 0) sh.esel = -1;
    __syncthreads();
    uint32_t kmax = 0, kmin = 0xffffffffu;
    int forced = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        kmax = max(kmax, (uint32_t)sh.wsum[0][w]);
        kmin = min(kmin, ~(uint32_t)sh.wsum[1][w]);
        forced += sh.wext[w];
    }
    // bits above `hi` are common to every ranked candidate (none ranked:
    // kmin > kmax, and every bit is left to the passes)
    const int cp = kmin <= kmax ? __clz((int)(kmin ^ kmax)) : 0;
    const int hi = max(32 - cp, 8);

    bool all = false;
    uint32_t pmask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
    uint32_t prefix = kmax & pmask;
    int wabove = forced;  // weight ranked above the current bucket
    for (int pass = 0;; ++pass) {
        const int shift = max(hi - 8 * (pass + 1), 0);
        int(*H)[256] = sh.hist[pass % 3];
        int *next = &sh.hist[(pass + 1) % 3][0][0];  // last read two passes ago
        for (int i = tid; i < 512; i += NT) next[i] = 0;
        // consecutive candidates mostly share a digit (scores of neighbouring
        // chunks have similar magnitude): a run of equal digits is added once,
        // by its last element (straight-line code, one predicated atomic per
        // element)
        bool m[PER];
        int dg[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            m[i] = cand[i] && (keys[i] & pmask) == prefix;
            dg[i] = (keys[i] >> shift) & 255u;
        }
        // after the first passes few candidates still match: a wave with none
        // skips the block
        bool any = false;
#pragma unroll
        for (int i = 0; i < PER; ++i) any = any || m[i];
        if (__ballot(any)) {
            int acc = 0;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                acc += m[i] ? wts[i] : 0;
                bool last = m[i];
                if (i + 1 < PER) last = last && !(m[i + 1] && dg[i + 1] == dg[i]);
                if (last) atomicAdd(&H[sub][dg[i]], acc);
                acc = last ? 0 : acc;
            }
        }
        __syncthreads();
        // every wave: lane l holds digits 255-4l .. 252-4l (descending)
        int h[4], s = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[j] = H[0][255 - 4 * lane - j] + H[1][255 - 4 * lane - j];
            s += h[j];
        }
        const int x = wave_scan_incl(s);
        if (pass == 0 && forced + __builtin_amdgcn_readlane(x, 63) <= bud) {  // everything fits
            all = true;
            break;
        }
        int before = wabove + x - s;  // weight of all higher digits
        int dsel = -1, bsel = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (before <= bud && before + h[j] > bud) {
                dsel = 255 - 4 * lane - j;
                bsel = before;
            }
            before += h[j];
        }
        // exactly one lane holds the crossing digit (the bucket's weight exceeds
        // what is left of the budget)
        const int src = max(__builtin_ffsll((long long)__ballot(dsel >= 0)) - 1, 0);
        const int digit = __builtin_amdgcn_readlane(dsel, src);
        wabove = __builtin_amdgcn_readlane(bsel, src);
        prefix |= uint32_t(digit) << shift;
        pmask |= 255u << shift;
        if (wabove == bud) {  // the cut is a digit boundary: nothing with this prefix is kept
            prefix |= ~pmask;
            pmask = 0xffffffffu;
            break;
        }
        if (shift == 0) break;  // every bit resolved
    }
    const uint32_t T = prefix;
    const int remaining = bud - wabove;

    // one scan of (count > T | count == T << 16, weight == T): ranks of the
    // kept candidates in index order
    bool gt[PER], eq[PER];
    int gtc = 0, eqc = 0, eqw = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool v = base + i < n;
        gt[i] = v && (all || keys[i] > T);
        eq[i] = v && !all && keys[i] == T;
        gtc += gt[i] ? 1 : 0;
        eqc += eq[i] ? 1 : 0;
        eqw += eq[i] ? wts[i] : 0;
    }
    int a = gtc | (eqc << 16), b = eqw, ta, tb;
    block_scan_pair<NT>(a, b, sh, ta, tb);
    a -= gtc | (eqc << 16);
    b -= eqw;
    int gt_before = a & 0xffff, eq_before = a >> 16;
    int e_sel;
    if (unit) {
        e_sel = min(ta >> 16, remaining);  // ties kept in index order while they fit
    } else {
        // the first candidate == T that no longer fits: its tie rank is the
        // number of ties kept (none such: every tie is kept).  At most one
        // thread finds it.
        int hit = -1;
        {
            int ce = eq_before, r = b;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                hit = (eq[i] && r <= remaining && r + wts[i] > remaining) ? ce : hit;
                r += eq[i] ? wts[i] : 0;
                ce += eq[i] ? 1 : 0;
            }
        }
        if (hit >= 0) sh.esel = hit;
        __syncthreads();
        e_sel = sh.esel < 0 ? (ta >> 16) : sh.esel;
    }
    begin(gt_before + min(eq_before, e_sel));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const bool keep = gt[i] || (eq[i] && eq_before < e_sel);
        emit(keep, gt_before + min(eq_before, e_sel), base + i, i);
        gt_before += gt[i] ? 1 : 0;
        eq_before += eq[i] ? 1 : 0;
    }
    (void)tb;
    return (ta & 0xffff) + e_sel;
}

// As above, writing the kept indices ascending to dst[0 .. min(count, dst_cap));
// returns min(count, dst_cap).
template <int NT, int PER>
__device__ __forceinline__ int radix_select_prefix(const uint32_t (&keys)[PER], const int (&wts)[PER], int base,
                                                   int n, int64_t budget, bool unit, int *dst, int dst_cap,
                                                   RadixShared &sh) {
    const int total = radix_select_prefix_emit<NT, PER>(
        keys, wts, base, n, budget, unit, [](int) {}, [&](bool keep, int pos, int idx, int) {
            if (keep && pos < dst_cap) dst[pos] = idx;
        }, sh);
    return min(total, dst_cap);
}

}  // namespace bsa
