// select.hip -- per-(sequence, KV head) chunk selection under a budget.
//
// Sources: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (keep the top-scoring chunks; budget =
// page_size x top_k tokens); "webarena" dataset README, section "Method
// configurations at a glance" (ratio budget max(1 + bos + eos,
// int(pages * ratio)) with forced first / last pages).  Variable chunks fill a
// token budget with the longest prefix of the score order that fits.
//
// All three budgets are one weighted radix select (radix_select.h) over the
// keys of select_rules.h: weight 1 per chunk for chunk budgets, the chunk
// length for token budgets.  One workgroup of 1024 threads per row, 2
// consecutive candidates per thread up to 2048 chunks, else 8 (up to 8192):
// the selection is a chain of short dependent steps, and 16 waves keep every
// SIMD busy while one waits.  The scores are requested before the row length
// is known (clamped into the row) so the two loads overlap.
#include "radix_select.h"
#include "select_rules.h"

namespace bsa {

template <int NT, int PER>
__global__ __launch_bounds__(NT) void select_kernel(const float *__restrict__ scores, KvView kv, ChunkView ch,
                                                        bsa_budget bud, int32_t *__restrict__ sel_idx,
                                                        int32_t *__restrict__ sel_count, int max_sel) {
    __shared__ RadixShared sh;
    args_ready(scores, kv.hkv, kv.seq_lens, kv.page, kv.log2page, ch.max_chunks, ch.starts, ch.num, bud.mode, bud.top_k,
               bud.tokens, bud.bos, bud.eos, bud.ratio);
    const int h = blockIdx.x, b = blockIdx.y;
    const float *row = scores + ((int64_t)b * kv.hkv + h) * ch.max_chunks;
    const int base = threadIdx.x * PER;
    float raw[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) raw[i] = row[min(base + i, ch.max_chunks - 1)];
    const int L = kv.seq_lens[b];
    const int n = ch.starts ? ch.num[b] : (L + kv.page - 1) >> kv.log2page;
    const RowBudget rb = row_budget(bud, n);
    uint32_t keys[PER];
    int wts[PER];
    select_keys<PER>(raw, base, n, rb, ch.starts ? ch.starts + (int64_t)b * (ch.max_chunks + 1) : nullptr, L,
                         kv.page, kv.log2page, keys, wts);
    int32_t *dst = sel_idx + ((int64_t)b * kv.hkv + h) * max_sel;
    const int cnt = radix_select_prefix<NT, PER>(keys, wts, base, n, rb.budget, !rb.tokens, dst, max_sel, sh);
    for (int i = cnt + threadIdx.x; i < max_sel; i += NT) dst[i] = -1;
    if (threadIdx.x == 0) sel_count[(int64_t)b * kv.hkv + h] = cnt;
}

hipError_t launch_select(const float *scores, const KvView &kv, const ChunkView &ch, const bsa_budget &b,
                         int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, hipStream_t s) {
    dim3 grid(kv.hkv, kv.batch);
    if (ch.max_chunks <= 1024 * 2)
        hipLaunchKernelGGL((select_kernel<1024, 2>), grid, dim3(1024), 0, s, scores, kv, ch, b, sel_idx, sel_count,
                           max_sel);
    else if (ch.max_chunks <= 1024 * 8)
        hipLaunchKernelGGL((select_kernel<1024, 8>), grid, dim3(1024), 0, s, scores, kv, ch, b, sel_idx, sel_count,
                           max_sel);
    else
        hipLaunchKernelGGL((select_kernel<1024, 16>), grid, dim3(1024), 0, s, scores, kv, ch, b, sel_idx, sel_count,
                           max_sel);
    return hipGetLastError();
}

}  // namespace bsa
