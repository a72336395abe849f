// select.hip -- per-(sequence, KV head) chunk selection under a budget.
//
// Sources: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (keep the top-scoring chunks; budget =
// page_size x top_k tokens); "webarena" dataset README, section "Method
// configurations at a glance" (ratio budget max(1 + bos + eos,
// int(pages * ratio)) with forced first / last pages).  Variable chunks fill a
// token budget with the longest prefix of the score order that fits.
//
// All three budgets are one weighted radix select (radix_select.h): weight 1
// per chunk for chunk budgets, the chunk length for token budgets.  Forced
// pages get the key 0xffffffff, above every finite score, so they are always
// part of the prefix and count inside K.  One workgroup per row (256 threads
// up to 2048 chunks, else 1024), 8 consecutive candidates per thread in
// registers (up to 8192 chunks).
#include "bsa_internal.h"
#include "radix_select.h"

namespace bsa {

constexpr int kSelPer = 8;

template <int NT>
__global__ __launch_bounds__(NT) void select_kernel(const float *__restrict__ scores, KvView kv, ChunkView ch,
                                                        bsa_budget bud, int32_t *__restrict__ sel_idx,
                                                        int32_t *__restrict__ sel_count, int max_sel) {
    __shared__ RadixShared sh;
    const int h = blockIdx.x, b = blockIdx.y;
    const int L = kv.seq_lens[b];
    const int n = ch.starts ? ch.num[b] : (L + kv.page - 1) >> kv.log2page;
    const float *row = scores + ((int64_t)b * kv.hkv + h) * ch.max_chunks;
    int64_t budget;
    bool forced_bos = false, forced_eos = false;
    const bool tokens = bud.mode == BSA_BUDGET_TOKENS;
    if (bud.mode == BSA_BUDGET_TOPK) {
        budget = bud.top_k;
    } else if (tokens) {
        budget = bud.tokens;
    } else {
        int64_t K = (int64_t)floor((double)n * bud.ratio);
        K = max(K, (int64_t)(1 + (bud.bos ? 1 : 0) + (bud.eos ? 1 : 0)));
        K = min(K, (int64_t)n);
        budget = K;
        forced_bos = bud.bos != 0;
        forced_eos = bud.eos != 0;
    }
    const int base = threadIdx.x * kSelPer;
    uint32_t keys[kSelPer];
    int wts[kSelPer];
    const int32_t *st = ch.starts ? ch.starts + (int64_t)b * (ch.max_chunks + 1) : nullptr;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
        const int c = base + i;
        keys[i] = 0u;
        wts[i] = 1;
        if (c < n) {
            uint32_t k = float_key(row[c]);
            if ((forced_bos && c == 0) || (forced_eos && c == n - 1)) k = 0xffffffffu;
            keys[i] = k;
            if (tokens) wts[i] = st ? st[c + 1] - st[c] : min(kv.page, L - (c << kv.log2page));
        }
    }
    int32_t *dst = sel_idx + ((int64_t)b * kv.hkv + h) * max_sel;
    const int cnt = radix_select_prefix<NT, kSelPer>(keys, wts, base, n, budget, dst, max_sel, sh);
    for (int i = cnt + threadIdx.x; i < max_sel; i += NT) dst[i] = -1;
    if (threadIdx.x == 0) sel_count[(int64_t)b * kv.hkv + h] = cnt;
}

hipError_t launch_select(const float *scores, const KvView &kv, const ChunkView &ch, const bsa_budget &b,
                         int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, hipStream_t s) {
    dim3 grid(kv.hkv, kv.batch);
    if (ch.max_chunks <= 256 * kSelPer)
        hipLaunchKernelGGL(select_kernel<256>, grid, dim3(256), 0, s, scores, kv, ch, b, sel_idx, sel_count, max_sel);
    else
        hipLaunchKernelGGL(select_kernel<1024>, grid, dim3(1024), 0, s, scores, kv, ch, b, sel_idx, sel_count,
                           max_sel);
    return hipGetLastError();
}

}  // namespace bsa
