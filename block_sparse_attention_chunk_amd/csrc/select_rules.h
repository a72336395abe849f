// select_rules.h -- the per-row selection rules shared by the selection
// kernel (select.hip) and the fused selection + decode kernel
// (select_decode.hip).  Internal to libbsa.
//
// Sources: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (keep the top-scoring chunks; budget =
// page_size x top_k tokens); "webarena" dataset README, section "Method
// configurations at a glance" (ratio budget max(1 + bos + eos,
// int(pages * ratio)) with forced first / last pages).  Variable chunks fill a
// token budget with the longest prefix of the score order that fits.
#pragma once

#include "bsa_internal.h"

namespace bsa {

struct RowBudget {
    int64_t budget;       // total weight the kept prefix may reach
    bool forced_bos, forced_eos;
    bool tokens;          // weights are chunk lengths (else 1 per chunk)
};

// The budget of one row of n chunks.
__device__ __forceinline__ RowBudget row_budget(const bsa_budget &bud, int n) {
    RowBudget r{0, false, false, bud.mode == BSA_BUDGET_TOKENS};
    if (bud.mode == BSA_BUDGET_TOPK) {
        r.budget = bud.top_k;
    } else if (r.tokens) {
        r.budget = bud.tokens;
    } else {
        int64_t K = (int64_t)floor((double)n * bud.ratio);
        K = max(K, (int64_t)(1 + (bud.bos ? 1 : 0) + (bud.eos ? 1 : 0)));
        r.budget = min(K, (int64_t)n);
        r.forced_bos = bud.bos != 0;
        r.forced_eos = bud.eos != 0;
    }
    return r;
}

// Keys and weights of candidates base .. base+PER-1 from their raw scores.
// Forced pages get the key 0xffffffff, above every finite score, so they are
// always part of the kept prefix and count inside K.  Token weights are the
// chunk's length: variable chunks from their starts, fixed pages clipped to
// the sequence end.  Candidates past n get key 0 and are ignored.
template <int PER>
__device__ __forceinline__ void select_keys(const float (&raw)[PER], int base, int n, const RowBudget &rb,
                                            const int32_t *starts, int L, int page, int log2page,
                                            uint32_t (&keys)[PER], int (&wts)[PER]) {
    // straight-line selects per candidate; only the token weights of variable
    // chunks need memory (uniform branch)
    const int fb = rb.forced_bos ? 0 : -1, fe = rb.forced_eos ? n - 1 : -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = base + i;
        const bool valid = c < n;
        const uint32_t k = (c == fb || c == fe) ? 0xffffffffu : float_key(raw[i]);
        keys[i] = valid ? k : 0u;
        wts[i] = 1;
    }
    if (rb.tokens) {
        if (starts) {
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int c = min(base + i, max(n - 1, 0));
                wts[i] = base + i < n ? starts[c + 1] - starts[c] : 1;
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER; ++i) wts[i] = base + i < n ? min(page, L - ((base + i) << log2page)) : 1;
        }
    }
}

}  // namespace bsa
