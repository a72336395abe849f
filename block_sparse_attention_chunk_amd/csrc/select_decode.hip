// select_decode.hip -- per-(sequence, KV head) chunk selection fused into the
// split-K decode attention, for fixed 16-token pages.
//
// Sources: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (score, keep the top chunks under the budget,
// attend only to them); "webarena" dataset README, section "Method
// configurations at a glance" (ratio budget with forced first / last pages).
//
// Every workgroup (KV split, KV head, sequence) reads the whole score row of
// its (sequence, KV head) -- a few KiB, mostly from L2 -- and runs the same
// weighted radix select as the selection kernel (identical rules, identical
// kept set).  The kept pages come out in ascending order; position p goes to
// split p mod splits, so each workgroup keeps only its own share in LDS, in
// the same order and with the same wave assignment as the unfused decode
// kernel at the same split count (so both give bit-identical outputs).  The
// block-table entries are read with the scores, so the kept pages carry their
// physical numbers and the attention starts its K/V reads without a lookup.
// The split-0 workgroup also writes the kept list and its length when asked.
// This removes one launch and the selection's round trips through memory from
// every decode step; the redundant per-split selection costs a few
// microseconds of on-chip work per workgroup.  When the grid has at most one
// workgroup per compute unit (a few sequences), that selection is the
// critical path, so 8 waves share it; the attention still runs on the first
// 4 waves with the unfused kernel's assignment.
#include "decode_common.h"
#include "radix_select.h"
#include "select_rules.h"

namespace bsa {

constexpr int kFusedListCap = 2048;  // kept pages per workgroup
constexpr int kSmallGrid = 256;      // workgroups: one per compute unit

template <typename T, int D, int GP, int PER, int NT>
__global__ __launch_bounds__(NT, (sizeof(T) == 2 && NT == 256) ? (PER >= 32 ? 2 : 3) : 1)
void select_decode_kernel(const T *__restrict__ q, int hq, KvView kv, const float *__restrict__ scores,
                          bsa_budget bud, int32_t *__restrict__ sel_idx, int32_t *__restrict__ sel_count,
                          int max_sel, float scale_log2, int splits, float *__restrict__ out,
                          float *__restrict__ part_o, float *__restrict__ part_ml) {
    constexpr int NW = DecTraits<T, D>::kNW, R = region_floats<D, GP>();
    __shared__ __attribute__((aligned(16))) float regions[kDecWaves * R];
    __shared__ float mbuf[kDecWaves * 16], lbuf[kDecWaves * 16];
    __shared__ RadixShared sh;
    __shared__ int32_t list[kFusedListCap], plist[kFusedListCap];  // logical / physical pages of this split
    args_ready(q, hq, kv.hkv, kv.max_pages, kv.bt, kv.seq_lens, scores, bud.mode, bud.top_k, bud.tokens, bud.bos,
               bud.eos, bud.ratio);
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int g = hq / kv.hkv;
    const int mc = kv.max_pages;

    // scores, q and the row length are requested together
    const float *row = scores + ((int64_t)b * kv.hkv + h) * mc;
    const int base = threadIdx.x * PER;
    float raw[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) raw[i] = row[min(base + i, mc - 1)];
    // the block-table entries of the same candidates, so the kept pages come
    // with their physical numbers and the attention needs no lookup
    // (without a block table the load reads the score row instead, so it stays
    // unconditional and the memory waits stay exact)
    const bool has_bt = kv.bt != nullptr;
    const int32_t *btr = has_bt ? kv.bt + (int64_t)b * kv.max_pages : reinterpret_cast<const int32_t *>(row);
    const int bt_mask = has_bt ? -1 : 0;  // a mask, not a select: a select would move the load into a branch
    int phys[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = min(base + i, mc - 1);
        phys[i] = (btr[c] & bt_mask) | ((b * kv.max_pages + c) & ~bt_mask);
    }
    uint4 qb[NW];
    load_q_operand<T, D>(q, hq, g, b, h, lane, qb);
    const int L = kv.seq_lens[b];
    const int n = (L + 15) >> 4;

    const RowBudget rb = row_budget(bud, n);
    uint32_t keys[PER];
    int wts[PER];
    select_keys<PER>(raw, base, n, rb, nullptr, L, 16, 4, keys, wts);
    int32_t *dst = (split == 0 && sel_idx) ? sel_idx + ((int64_t)b * kv.hkv + h) * max_sel : nullptr;
    // rank p goes to split p mod splits, slot p / splits; a thread's kept pages
    // have consecutive ranks, so one division per thread sets (slot, split)
    // and each kept page steps it
    int qs = 0, rs = 0;
    const int cnt = radix_select_prefix_emit<NT, PER>(
        keys, wts, base, n, rb.budget, !rb.tokens,
        [&](int p0) {
            qs = p0 / splits;
            rs = p0 - qs * splits;
        },
        [&](bool keep, int pos, int idx, int i) {
            if (dst && keep && pos < max_sel) dst[pos] = idx;
            if (keep && rs == split) {  // qs < kFusedListCap (host-checked)
                list[qs] = idx;
                plist[qs] = phys[i];
            }
            rs += keep ? 1 : 0;
            const bool wrap = rs == splits;
            rs = wrap ? 0 : rs;
            qs += wrap ? 1 : 0;
        },
        sh);
    if (dst) {
        for (int i = cnt + (int)threadIdx.x; i < max_sel; i += NT) dst[i] = -1;
        if (threadIdx.x == 0) sel_count[(int64_t)b * kv.hkv + h] = min(cnt, max_sel);
    }
    __syncthreads();

    // this workgroup's items: local positions w, w + 4, ... of its list, for
    // the first kDecWaves waves (the others only helped with the selection)
    const int local = cnt > split ? (cnt - split + splits - 1) / splits : 0;
    const int n_mine = (w < kDecWaves && local > w) ? (local - w + kDecWaves - 1) / kDecWaves : 0;
    WaveState<T, D, GP> st;
    init_state(st);
    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
    const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
    auto slot = [&](int ib) { return min(w + kDecWaves * (ib + lane), kFusedListCap - 1); };
    auto page_of = [&](int ib) { return list[slot(ib)]; };
    auto phys_of = [&](int ib, int) { return plist[slot(ib)]; };
    if (w < kDecWaves)
        stream_pages<T, D, GP, BSA_DECODE_PD>(st, qb, kv, kb, vb, L, n_mine, page_of, phys_of, scale_log2,
                                              regions + w * R, lane);
    finish_workgroup<T, D, GP, NT>(st, regions, mbuf, lbuf, g, hq, b, h, split, splits, out, part_o, part_ml);
}

template <typename T, int D, int GP>
static void launch_sd_t(const void *q, int hq, const KvView &kv, const float *scores, const bsa_budget &bud,
                        int32_t *sel_idx, int32_t *sel_count, int max_sel, float scale_log2, int splits, float *out,
                        float *part_o, float *part_ml, hipStream_t s) {
    dim3 grid(splits, kv.hkv, kv.batch);
#define BSA_SD_LAUNCH(PER, NT)                                                                                    \
    hipLaunchKernelGGL((select_decode_kernel<T, D, GP, PER, NT>), grid, dim3(NT), 0, s, (const T *)q, hq, kv, scores, \
                       bud, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o, part_ml)
    // A grid of at most one workgroup per compute unit is latency-bound: 8
    // waves share the selection (half the candidates per thread), and the
    // first 4 attend as usual.  Larger grids keep 4 waves, so 3 workgroups fit
    // on a compute unit (2 with 32 candidates per thread, whose registers
    // would otherwise spill).
    const int64_t wgs = (int64_t)splits * kv.hkv * kv.batch;
    if (wgs <= kSmallGrid) {
        if (kv.max_pages <= 512 * 4)
            BSA_SD_LAUNCH(4, 512);
        else if (kv.max_pages <= 512 * 8)
            BSA_SD_LAUNCH(8, 512);
        else
            BSA_SD_LAUNCH(16, 512);
    } else {
        if (kv.max_pages <= 256 * 8)
            BSA_SD_LAUNCH(8, 256);
        else if (kv.max_pages <= 256 * 16)
            BSA_SD_LAUNCH(16, 256);
        else
            BSA_SD_LAUNCH(32, 256);
    }
#undef BSA_SD_LAUNCH
}

template <typename T, int D>
static void launch_sd_g(const void *q, int hq, const KvView &kv, const float *scores, const bsa_budget &bud,
                        int32_t *sel_idx, int32_t *sel_count, int max_sel, float scale_log2, int splits, float *out,
                        float *part_o, float *part_ml, hipStream_t s) {
    const int g = hq / kv.hkv;
    if (g <= 4)
        launch_sd_t<T, D, 4>(q, hq, kv, scores, bud, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                             part_ml, s);
    else if (g <= 8)
        launch_sd_t<T, D, 8>(q, hq, kv, scores, bud, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                             part_ml, s);
    else
        launch_sd_t<T, D, 16>(q, hq, kv, scores, bud, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                              part_ml, s);
}

hipError_t launch_select_decode(const void *q, int32_t hq, const KvView &kv, const float *scores,
                                const bsa_budget &bud, int32_t *sel_idx, int32_t *sel_count, int32_t max_sel,
                                float scale, int32_t splits, float *out, void *ws, hipStream_t s) {
    const float scale_log2 = scale * kLog2e;
    float *part_o = nullptr, *part_ml = nullptr;
    if (splits > 1) {
        part_o = (float *)ws;
        part_ml = part_o + (size_t)kv.batch * hq * splits * kv.d;
    }
    if (kv.dtype == BSA_BF16) {
        if (kv.d == 128)
            launch_sd_g<uint16_t, 128>(q, hq, kv, scores, bud, sel_idx, sel_count, max_sel, scale_log2, splits, out,
                                       part_o, part_ml, s);
        else
            launch_sd_g<uint16_t, 64>(q, hq, kv, scores, bud, sel_idx, sel_count, max_sel, scale_log2, splits, out,
                                      part_o, part_ml, s);
    } else {
        if (kv.d == 128)
            launch_sd_g<float, 128>(q, hq, kv, scores, bud, sel_idx, sel_count, max_sel, scale_log2, splits, out,
                                    part_o, part_ml, s);
        else
            launch_sd_g<float, 64>(q, hq, kv, scores, bud, sel_idx, sel_count, max_sel, scale_log2, splits, out,
                                   part_o, part_ml, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1 || !out) return e;  // no out: the partials are the result
    return launch_decode_merge(splits, part_o, part_ml, out, hq, kv.batch, kv.d, s);
}

}  // namespace bsa
