// select.hip -- per-(sequence, KV head) chunk selection under a budget.
//
// Sources: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (keep the top-scoring chunks; budget =
// page_size x top_k tokens); "webarena" dataset README, section "Method
// configurations at a glance" (ratio budget max(1 + bos + eos,
// int(pages * ratio)) with forced first / last pages).  Variable chunks fill a
// token budget with the longest prefix of the score order that fits.
//
// All three budgets are one weighted radix select.  Candidates are ordered by
// (score descending, index ascending); with a weight per candidate (1 for
// chunk counts, the chunk length for token budgets) the selection is the
// longest prefix of that order whose total weight <= budget.  Four 8-bit
// passes over order-preserving float keys find the key T of the first
// candidate that does not fit; every key > T is kept, and the candidates with
// key == T are kept in ascending index order while their running weight fits.
// Forced pages get the key 0xffffffff, above every finite score.  The output
// is written in ascending index order by a block-wide scan, so ties need no
// sort.  One 256-thread workgroup per row; the keys live in LDS.
#include "bsa_internal.h"
#include "radix_select.h"

namespace bsa {

__device__ __forceinline__ int chunk_weight(const KvView &kv, const ChunkView &ch, int b, int L, int i,
                                            bool tokens) {
    if (!tokens) return 1;
    if (ch.starts) {
        const int32_t *st = ch.starts + (int64_t)b * (ch.max_chunks + 1);
        return st[i + 1] - st[i];
    }
    const int s = i << kv.log2page;
    return min(kv.page, L - s);
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float *__restrict__ scores, KvView kv,
                                                             ChunkView ch, bsa_budget bud, int32_t *__restrict__ sel_idx,
                                                             int32_t *__restrict__ sel_count, int max_sel) {
    extern __shared__ uint32_t keys[];
    __shared__ int hist[256];
    __shared__ int scan[8];
    __shared__ int bcast[2];
    const int h = blockIdx.x, b = blockIdx.y;
    const int L = kv.seq_lens[b];
    const int n = ch.starts ? ch.num[b] : (L + kv.page - 1) >> kv.log2page;
    const float *row = scores + ((int64_t)b * kv.hkv + h) * ch.max_chunks;
    int64_t budget;
    bool forced_bos = false, forced_eos = false;
    if (bud.mode == BSA_BUDGET_TOPK) {
        budget = bud.top_k;
    } else if (bud.mode == BSA_BUDGET_TOKENS) {
        budget = bud.tokens;
    } else {
        int64_t K = (int64_t)floor((double)n * bud.ratio);
        K = max(K, (int64_t)(1 + (bud.bos ? 1 : 0) + (bud.eos ? 1 : 0)));
        K = min(K, (int64_t)n);
        budget = K;
        forced_bos = bud.bos != 0;
        forced_eos = bud.eos != 0;
    }
    for (int i = threadIdx.x; i < n; i += kSelThreads) {
        uint32_t k = float_key(row[i]);
        if ((forced_bos && i == 0) || (forced_eos && i == n - 1)) k = 0xffffffffu;
        keys[i] = k;
    }
    __syncthreads();
    const bool tokens = bud.mode == BSA_BUDGET_TOKENS;
    int32_t *dst = sel_idx + ((int64_t)b * kv.hkv + h) * max_sel;
    auto weight = [&](int i) { return chunk_weight(kv, ch, b, L, i, tokens); };
    const int cnt = radix_select_prefix(keys, n, budget, weight, dst, max_sel, hist, scan, bcast);
    for (int i = cnt + threadIdx.x; i < max_sel; i += kSelThreads) dst[i] = -1;
    if (threadIdx.x == 0) sel_count[(int64_t)b * kv.hkv + h] = cnt;
}

hipError_t launch_select(const float *scores, const KvView &kv, const ChunkView &ch, const bsa_budget &b,
                         int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, hipStream_t s) {
    dim3 grid(kv.hkv, kv.batch), block(kSelThreads);
    const size_t lds = (size_t)ch.max_chunks * sizeof(uint32_t);
    hipLaunchKernelGGL(select_kernel, grid, block, lds, s, scores, kv, ch, b, sel_idx, sel_count, max_sel);
    return hipGetLastError();
}

}  // namespace bsa
