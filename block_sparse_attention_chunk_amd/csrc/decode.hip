// decode.hip -- split-K online-softmax attention of one decode query per
// sequence over the selected chunks of a paged GQA KV cache, plus the merge.
//
// Source: "Sparse Attention for Web Agents -- Offline Replay Records",
// section "The comparison" (attend only to the kept chunks; the budget is the
// number of KV tokens attended).  The split-K form with a final merge of the
// (max, sum, output) partials is this library's design.
//
// One workgroup (4 waves) per (KV split, KV head, sequence) serves the whole
// GQA group, so every selected K/V page is read from HBM once for all
// H_q/H_kv query heads.  A wave consumes one 16-token segment at a time:
//   * S = K_seg . Q_group^T on the matrix cores (v_mfma_f32_16x16x32_bf16):
//     token rows x 16 (zero-padded) query-head columns.  Each lane loads a
//     contiguous D/4-element slice of its token row (16-byte loads covering
//     the 4 KiB page), and K and Q split the reduction over D the same way, so
//     the pairing needs no particular k order;
//   * online softmax per head in fp32 (log2 domain) straight from the MFMA
//     accumulators (lane = head, 4 tokens per lane);
//   * O^T += V^T . P on the matrix cores (v_mfma_f32_16x16x16_bf16): each lane
//     loads 4 token rows x D/16 consecutive dims of V with one 16-byte load per
//     row (a quarter-wave reads a whole 256-byte row), and the output tile's
//     row index is mapped to dims so that these registers already are the A
//     operand (no transpose); P (still in registers, laid out exactly as the
//     B operand needs) is split into bf16 hi + lo parts, so the product keeps
//     ~16 bits of P (relative error ~2^-17).
// Each wave loads its page numbers up front (one per lane, read back with
// readlane) and prefetches unconditionally, so the memory counters stay exact
// and BSA_DECODE_PD pages are always in flight while the current one is
// consumed.  The 4 waves' partials are merged in LDS; with more than one
// split a small kernel merges the splits (a kernel boundary is the cheap way to
// make the partials of all XCDs visible).  HBM-bound.
//
// float32 caches use the same structure with 16x16x4 f32 MFMAs for S and the
// vector ALU for P . V.  Large batches of 16-token pages can instead take the
// balanced schedule further down (equal shares of all rows' pages, one
// workgroup per compute unit), with the same per-page machinery.
#include "decode_common.h"
#include "radix_select.h"

namespace bsa {

// Fixed 16-token pages: one item = one page.  PD pages are in flight per wave
// while the current one is consumed.
template <typename T, int D, int GP, int PD>
__global__ __launch_bounds__(256, (sizeof(T) == 2 && PD == 1) ? 3 : (sizeof(T) == 2 ? 2 : 1))
void decode_paged16_kernel(const T *__restrict__ q, int hq, KvView kv, const int32_t *__restrict__ sel_idx,
                           const int32_t *__restrict__ sel_count, int max_sel, float scale_log2, int splits,
                           float *__restrict__ out, float *__restrict__ part_o, float *__restrict__ part_ml) {
    constexpr int NW = DecTraits<T, D>::kNW, R = region_floats<D, GP>();
    __shared__ __attribute__((aligned(16))) float regions[kDecWaves * R];
    __shared__ float mbuf[kDecWaves * 16], lbuf[kDecWaves * 16];
    args_ready(q, hq, kv.hkv, kv.bt, kv.seq_lens, kv.max_pages, sel_idx, sel_count, max_sel, splits);
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int g = hq / kv.hkv;
    const int32_t *items = sel_idx ? sel_idx + ((int64_t)b * kv.hkv + h) * max_sel : nullptr;
    // Items are dealt to splits and waves round-robin: wave w of split s takes
    // items s + splits * (w + 4 j).  The indices do not depend on the item
    // count, so the first 64 of this wave's page numbers are requested at once,
    // clamped into the row, in parallel with the count.
    const int wstride = splits * kDecWaves;
    const int first = split + splits * w;
    int spec = first + wstride * lane;
    // The page numbers, the item count, the row length and the query are
    // requested together, unconditionally (without a selection the spare
    // loads read the row length), and waited for once.
    const int32_t *spec_src = items ? items : kv.seq_lens;
    int spec_ld = spec_src[items ? min(spec, max_sel - 1) : b];
    const int32_t *cnt_src = sel_idx ? sel_count + ((int64_t)b * kv.hkv + h) : kv.seq_lens + b;
    int cnt_ld = *cnt_src;
    int len_ld = kv.seq_lens[b];
    uint4 qb[NW];
    load_q_operand<T, D>(q, hq, g, b, h, lane, qb);
    asm volatile("" : "+v"(spec_ld), "+v"(cnt_ld), "+v"(len_ld)::"memory");
    const int L = __builtin_amdgcn_readfirstlane(len_ld);
    const int npages = (L + 15) >> 4;
    // kept page ids come from the caller: an id outside the row is clamped
    // into it (wrong values, no stray address) rather than dereferenced
    const int last_page = max(npages - 1, 0);
    if (items) spec = min(max(spec_ld, 0), last_page);
    const int nitems = sel_idx ? min(max(__builtin_amdgcn_readfirstlane(cnt_ld), 0), max_sel) : npages;
    WaveState<T, D, GP> st;
    init_state(st);

    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
    const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
    const int32_t *bt = kv.bt ? kv.bt + (int64_t)b * kv.max_pages : nullptr;
    float *region = regions + w * R;

    const int n_mine = first < nitems ? (nitems - first + wstride - 1) / wstride : 0;
    auto page_of = [&](int base) {
        if (base == 0) return spec;
        const int it = first + wstride * (base + (int)(threadIdx.x & 63));
        return items ? min(max(items[min(it, max_sel - 1)], 0), last_page) : it;
    };
    auto phys_of = [&](int, int page) { return bt ? bt[page] : b * kv.max_pages + page; };
    stream_pages<T, D, GP, PD>(st, qb, kv, kb, vb, L, n_mine, page_of, phys_of, scale_log2, region, lane);
    finish_workgroup<T, D, GP>(st, regions, mbuf, lbuf, g, hq, b, h, split, splits, out, part_o, part_ml);
}

// Per-token fallback for what the segment kernel below does not take: pages
// under 16 tokens (a 16-token segment may span more than two of them) and rows
// of more than 2048 kept chunks.  Each split takes a contiguous range of the
// row's chunks, and a wave consumes one chunk at a time in 16-token segments
// with a block-table lookup per lane; only the segment's valid rows are read.
template <typename T, int D, int GP>
__global__ __launch_bounds__(256) void decode_chunked_kernel(const T *__restrict__ q, int hq, KvView kv, ChunkView ch,
                                                             const int32_t *__restrict__ sel_idx,
                                                             const int32_t *__restrict__ sel_count, int max_sel,
                                                             float scale_log2, int splits, float *__restrict__ out,
                                                             float *__restrict__ part_o, float *__restrict__ part_ml) {
    using Tr = DecTraits<T, D>;
    constexpr int NW = Tr::kNW, VR = Tr::kVRegs, R = region_floats<D, GP>();
    __shared__ __attribute__((aligned(16))) float regions[kDecWaves * R];
    __shared__ float mbuf[kDecWaves * 16], lbuf[kDecWaves * 16];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n16 = lane & 15, G = lane >> 4;
    const int g = hq / kv.hkv;
    const int L = kv.seq_lens[b];
    const int nch = ch.starts ? ch.num[b] : (L + kv.page - 1) >> kv.log2page;
    const int nitems = sel_idx ? min(max(sel_count[(int64_t)b * kv.hkv + h], 0), max_sel) : nch;
    const int32_t *items = sel_idx ? sel_idx + ((int64_t)b * kv.hkv + h) * max_sel : nullptr;
    const int i0 = (int)((int64_t)split * nitems / splits), i1 = (int)((int64_t)(split + 1) * nitems / splits);

    uint4 qb[NW];
    load_q_operand<T, D>(q, hq, g, b, h, lane, qb);
    WaveState<T, D, GP> st;
    init_state(st);

    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
    const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
    const int32_t *bt = kv.bt ? kv.bt + (int64_t)b * kv.max_pages : nullptr;
    auto row_of = [&](const T *base, int tok) {
        const int page = tok >> kv.log2page, slot = tok & (kv.page - 1);
        const int64_t phys = bt ? bt[page] : (int64_t)b * kv.max_pages + page;
        return base + phys * kv.sp + (int64_t)slot * kv.st;
    };
    float *region = regions + w * R;
    for (int it = i0 + w; it < i1; it += kDecWaves) {
        // a caller's chunk id outside the row is clamped into it
        const int c = __builtin_amdgcn_readfirstlane(items ? min(max(items[it], 0), max(nch - 1, 0)) : it);
        int s, e;
        if (ch.starts) {
            s = ch.starts[(int64_t)b * (ch.max_chunks + 1) + c];
            e = ch.starts[(int64_t)b * (ch.max_chunks + 1) + c + 1];
        } else {
            s = c << kv.log2page;
            e = min(s + kv.page, L);
        }
        for (int t0 = s; t0 < e; t0 += 16) {
            const int valid = min(16, e - t0);
            uint4 ks[NW];
            uint32_t vr[VR];
            if (n16 < valid) {
                load_k_slice<T, D>(row_of(kb, t0 + n16), ks, G);
            } else {
#pragma unroll
                for (int i = 0; i < NW; ++i) ks[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < VR / Tr::kRowRegs; ++r) {
                const int t = v_token<T, D>(r, G);
                if (t < valid) {
                    load_v_row<T, D>(row_of(vb, t0 + t), vr + r * Tr::kRowRegs, lane);
                } else {
#pragma unroll
                    for (int c2 = 0; c2 < Tr::kRowRegs; ++c2) vr[r * Tr::kRowRegs + c2] = 0u;
                }
            }
            consume<T, D, GP>(st, ks, vr, qb, valid, scale_log2, region, lane);
        }
    }
    finish_workgroup<T, D, GP>(st, regions, mbuf, lbuf, g, hq, b, h, split, splits, out, part_o, part_ml);
}

// General chunks cut into 16-token segments: variable token intervals, or
// fixed pages of 16 tokens or more.  The workgroup first lays out the
// segments of its row's kept chunks: each thread takes kSegItems / 256
// consecutive chunks, and one block scan of their segment counts gives every
// chunk its first segment number and its token range in LDS.  Segments are
// then dealt to splits and waves round-robin like pages (segment n goes to
// split n mod splits), so the work of a row spreads evenly whatever the chunk
// lengths.  A wave looks up 64 of its segments at once, one per lane (binary
// search in LDS, then the physical page of the segment's first and last token
// from the block table: a segment of >= 16-token pages spans at most two), and
// streams them with one segment in flight, reading the lane's values back with
// readlane.  Rows past a segment's end are clamped onto its last row and
// masked.
constexpr int kSegItems = 2048;  // kept chunks per (sequence, KV head) laid out in LDS

template <typename T, int D, int GP>
__global__ __launch_bounds__(256, 2) void decode_segments_kernel(const T *__restrict__ q, int hq, KvView kv,
                                                                 ChunkView ch, const int32_t *__restrict__ sel_idx,
                                                                 const int32_t *__restrict__ sel_count, int max_sel,
                                                                 float scale_log2, int splits,
                                                                 float *__restrict__ out, float *__restrict__ part_o,
                                                                 float *__restrict__ part_ml) {
    using Tr = DecTraits<T, D>;
    constexpr int NW = Tr::kNW, VR = Tr::kVRegs, R = region_floats<D, GP>();
    constexpr int PER = kSegItems / 256, PD = 1, NB = PD + 1;
    __shared__ __attribute__((aligned(16))) float regions[kDecWaves * R];
    __shared__ float mbuf[kDecWaves * 16], lbuf[kDecWaves * 16];
    __shared__ int seg_first[kSegItems], tok_begin[kSegItems], tok_end[kSegItems];
    __shared__ int wtot[kDecWaves];
    args_ready(q, hq, kv.hkv, kv.seq_lens, ch.starts, ch.num, sel_idx, sel_count, max_sel, splits);
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n16 = lane & 15, G = lane >> 4;
    const int g = hq / kv.hkv;
    const int L = kv.seq_lens[b];
    const int nch = ch.starts ? ch.num[b] : (L + kv.page - 1) >> kv.log2page;
    // the kept chunks (<= kSegItems: host-checked against max_sel / max_chunks)
    const int nitems = min(sel_idx ? min(max(sel_count[(int64_t)b * kv.hkv + h], 0), max_sel) : nch, kSegItems);
    const int32_t *items = sel_idx ? sel_idx + ((int64_t)b * kv.hkv + h) * max_sel : nullptr;
    const int32_t *cs = ch.starts ? ch.starts + (int64_t)b * (ch.max_chunks + 1) : nullptr;

    uint4 qb[NW];
    load_q_operand<T, D>(q, hq, g, b, h, lane, qb);

    // token ranges and segment counts of this thread's chunks, then the block
    // scan of the counts
    int tb[PER], te[PER], before[PER], run = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = threadIdx.x * PER + k;
        int s0 = 0, e0 = 0;
        if (i < nitems) {
            const int c = items ? min(max(items[i], 0), max(nch - 1, 0)) : i;   // caller ids clamped into the row
            if (cs) {
                s0 = cs[c];
                e0 = cs[c + 1];
            } else {
                s0 = c << kv.log2page;
                e0 = s0 + kv.page;
            }
            e0 = min(e0, L);
            s0 = min(s0, e0);
        }
        tb[k] = s0, te[k] = e0, before[k] = run;
        run += (e0 - s0 + 15) >> 4;
    }
    const int incl = wave_scan_incl(run);
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    int woff = 0, total = 0;
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x) {
        woff += x < w ? wtot[x] : 0;
        total += wtot[x];
    }
    const int excl = woff + incl - run;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = threadIdx.x * PER + k;
        if (i < nitems) {
            seg_first[i] = excl + before[k];
            tok_begin[i] = tb[k];
            tok_end[i] = te[k];
        }
    }
    __syncthreads();

    WaveState<T, D, GP> st;
    init_state(st);
    const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
    const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
    const int32_t *bt = kv.bt ? kv.bt + (int64_t)b * kv.max_pages : nullptr;
    float *region = regions + w * R;
    const int wstride = splits * kDecWaves, first = split + splits * w;
    const int n_mine = first < total ? (total - first + wstride - 1) / wstride : 0;

    for (int base = 0; base < n_mine; base += 64) {
        const int cnt = min(64, n_mine - base);
        // lane l: the wave's segment base + l (clamped to the last one)
        int my_t0, my_valid, my_p0, my_p1;
        {
            const int gs = first + wstride * (base + min(lane, cnt - 1));
            int lo = 0;  // the last chunk whose first segment is <= gs
#pragma unroll
            for (int step = kSegItems / 2; step > 0; step >>= 1)
                if (lo + step < nitems && seg_first[lo + step] <= gs) lo += step;
            my_t0 = tok_begin[lo] + 16 * (gs - seg_first[lo]);
            my_valid = min(16, tok_end[lo] - my_t0);
            const int pa = my_t0 >> kv.log2page, pz = (my_t0 + my_valid - 1) >> kv.log2page;
            my_p0 = bt ? bt[pa] : b * kv.max_pages + pa;
            my_p1 = bt ? bt[pz] : b * kv.max_pages + pz;
        }
        auto issue = [&](int j, uint4 (&ks)[NW], uint32_t (&vr)[VR], int &valid) {
            const int t0 = __builtin_amdgcn_readlane(my_t0, j), vl = __builtin_amdgcn_readlane(my_valid, j);
            const int p0 = __builtin_amdgcn_readlane(my_p0, j), p1 = __builtin_amdgcn_readlane(my_p1, j);
            const int pg0 = t0 >> kv.log2page;
            valid = vl;
            auto row = [&](const T *base_ptr, int slot) {
                const int tok = t0 + min(slot, vl - 1);
                const int phys = (tok >> kv.log2page) == pg0 ? p0 : p1;
                return base_ptr + (int64_t)phys * kv.sp + (int64_t)(tok & (kv.page - 1)) * kv.st;
            };
            load_k_slice<T, D>(row(kb, n16), ks, G);
#pragma unroll
            for (int r = 0; r < VR / Tr::kRowRegs; ++r)
                load_v_row<T, D>(row(vb, v_token<T, D>(r, G)), vr + r * Tr::kRowRegs, lane);
        };
        auto clear_tail = [&](uint32_t (&vr)[VR], int valid) {
#pragma unroll
            for (int r = 0; r < VR / Tr::kRowRegs; ++r)
#pragma unroll
                for (int c = 0; c < Tr::kRowRegs; ++c)
                    vr[r * Tr::kRowRegs + c] = v_token<T, D>(r, G) < valid ? vr[r * Tr::kRowRegs + c] : 0u;
        };
        uint4 ks[NB][NW];
        uint32_t vr[NB][VR];
        int valid[NB];
#pragma unroll
        for (int s = 0; s < PD; ++s) issue(min(s, cnt - 1), ks[s], vr[s], valid[s]);
        // whole rounds of NB segments, then the ones still in flight; no early
        // exit inside a round, so the counter waits stay exact
        const int full = cnt - cnt % NB;
        for (int j = 0; j < full; j += NB) {
#pragma unroll
            for (int s = 0; s < NB; ++s) {
                const int sn = (s + PD) % NB;
                issue(min(j + s + PD, cnt - 1), ks[sn], vr[sn], valid[sn]);
                __builtin_amdgcn_sched_barrier(0);  // the prefetch stays ahead of the consumption
                clear_tail(vr[s], valid[s]);
                consume<T, D, GP>(st, ks[s], vr[s], qb, valid[s], scale_log2, region, lane);
            }
        }
#pragma unroll
        for (int s = 0; s < PD; ++s) {
            if (full + s < cnt) {
                clear_tail(vr[s], valid[s]);
                consume<T, D, GP>(st, ks[s], vr[s], qb, valid[s], scale_log2, region, lane);
            }
        }
    }
    finish_workgroup<T, D, GP>(st, regions, mbuf, lbuf, g, hq, b, h, split, splits, out, part_o, part_ml);
}

// Balanced schedule for batches (16-token pages, selected items).  With a
// fixed split count per row, rows of unequal length leave the compute units
// that hold short rows idle while the long ones finish, and one compute unit
// streams pages at a roughly fixed rate whatever the number of its
// workgroups, so the step lasts as long as its busiest unit.  Here the rows'
// kept pages are laid end to end (row r = b * H_kv + h holds positions
// [P_r, P_r + n_r)) and cut into kBalWgs equal shares of qn positions: one
// workgroup per compute unit, each streaming the same number of pages.  A
// share that crosses row ends yields one segment per row, each finished as a
// partial of its own; the partial of (row r, workgroup w) is entry r + w of
// the workspace (rows and shares both advance with position, so no two
// segments share an entry, and the entries of one row are consecutive).
__device__ __forceinline__ int bal_quantum(int total) {
    return max((total + kBalWgs - 1) / kBalWgs, kBalMinItems);
}

__device__ __forceinline__ int bal_count(const int32_t *sel_count, int r, int max_sel) {
    return min(max(sel_count[r], 0), max_sel);
}

__device__ __forceinline__ int wave_isum_all(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// One workgroup per compute unit: the register budget of one wave per SIMD.
template <typename T, int D, int GP, int PD>
__global__ __launch_bounds__(256, 1)
void decode_balanced_kernel(const T *__restrict__ q, int hq, KvView kv, const int32_t *__restrict__ sel_idx,
                            const int32_t *__restrict__ sel_count, int max_sel, float scale_log2,
                            float *__restrict__ part_o, float *__restrict__ part_ml) {
    constexpr int NW = DecTraits<T, D>::kNW, R = region_floats<D, GP>();
    __shared__ __attribute__((aligned(16))) float regions[kDecWaves * R];
    __shared__ float mbuf[kDecWaves * 16], lbuf[kDecWaves * 16];
    __shared__ int pre[kBalMaxRows + 1];
    __shared__ int wtot[kDecWaves];
    args_ready(q, hq, kv.hkv, kv.bt, kv.seq_lens, kv.max_pages, sel_idx, sel_count, max_sel);
    const int rows = kv.batch * kv.hkv;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int g = hq / kv.hkv;

    // 1. pre[r] = P_r (exclusive prefix of the clamped counts), pre[rows] = T:
    //    the counts are staged in LDS, then scanned 256 rows at a time
#pragma unroll 4
    for (int r = threadIdx.x; r < rows; r += kDecWaves * 64) pre[r] = bal_count(sel_count, r, max_sel);
    __syncthreads();
    int carry = 0;
    for (int base = 0; base < rows; base += kDecWaves * 64) {
        const int r = base + (int)threadIdx.x;
        const int c = r < rows ? pre[r] : 0;
        int inc = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o);
            inc += lane >= o ? y : 0;
        }
        if (lane == 63) wtot[w] = inc;
        __syncthreads();
        int off = carry;
        for (int k = 0; k < w; ++k) off += wtot[k];
        if (r < rows) pre[r] = off + inc - c;
        carry += wtot[0] + wtot[1] + wtot[2] + wtot[3];
        __syncthreads();  // wtot is rewritten by the next round
    }
    if (threadIdx.x == 0) pre[rows] = carry;
    __syncthreads();

    // 2. this workgroup's share and the row holding its first position
    const int total = __builtin_amdgcn_readfirstlane(pre[rows]);
    const int qn = bal_quantum(total);
    const int start = (int)blockIdx.x * qn;
    if (start >= total) return;
    const int end = min(start + qn, total);
    int lo = 0, hi = rows - 1;  // the last row r with P_r <= start (it holds start)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= start) lo = mid;
        else hi = mid - 1;
    }
    lo = __builtin_amdgcn_readfirstlane(lo);

    // 3. one segment per row met: items [a, e) of row r, wave w taking a + w + 4 j
    for (int r = lo; r < rows; ++r) {
        const int p0 = __builtin_amdgcn_readfirstlane(pre[r]), p1 = __builtin_amdgcn_readfirstlane(pre[r + 1]);
        if (p0 >= end) break;
        const int a = max(start, p0) - p0, e = min(end, p1) - p0;
        if (e <= a) continue;  // an empty row
        const int b = r / kv.hkv, h = r - b * kv.hkv;
        const int32_t *items = sel_idx + (int64_t)r * max_sel;
        const int first = a + w, n = e - a;
        const int n_mine = n > w ? (n - w + kDecWaves - 1) / kDecWaves : 0;
        // the first 64 page numbers, the row length and the query, waited for once
        int spec = items[min(first + kDecWaves * lane, max_sel - 1)];
        int len_ld = kv.seq_lens[b];
        uint4 qb[NW];
        load_q_operand<T, D>(q, hq, g, b, h, lane, qb);
        asm volatile("" : "+v"(spec), "+v"(len_ld)::"memory");
        const int L = __builtin_amdgcn_readfirstlane(len_ld);
        const int last_page = max(((L + 15) >> 4) - 1, 0);   // caller page ids are clamped into the row
        spec = min(max(spec, 0), last_page);
        WaveState<T, D, GP> st;
        init_state(st);
        const T *kb = reinterpret_cast<const T *>(kv.k) + (int64_t)h * kv.sh;
        const T *vb = reinterpret_cast<const T *>(kv.v) + (int64_t)h * kv.sh;
        const int32_t *bt = kv.bt ? kv.bt + (int64_t)b * kv.max_pages : nullptr;
        auto page_of = [&](int base) {
            if (base == 0) return spec;
            return min(max(items[min(first + kDecWaves * (base + (int)(threadIdx.x & 63)), max_sel - 1)], 0),
                       last_page);
        };
        auto phys_of = [&](int, int page) { return bt ? bt[page] : b * kv.max_pages + page; };
        stream_pages<T, D, GP, PD>(st, qb, kv, kb, vb, L, n_mine, page_of, phys_of, scale_log2, regions + w * R,
                                   lane);
        finish_workgroup_at<T, D, GP>(st, regions, mbuf, lbuf, g, 0, (int64_t)(r + (int)blockIdx.x) * g, 1,
                                      nullptr, part_o, part_ml);
        __syncthreads();  // the regions are reused by the next segment
    }
}

// Merge of the balanced schedule's segments of one (sequence, query head):
// the same weighted sum as decode_merge_kernel below, over the consecutive
// entries the row's positions fall into (recomputed from the counts exactly
// as the attention kernel cut them).  A row with no kept item has no entry
// and gets 0/0, as the split path does.
template <int D>
__global__ __launch_bounds__(64) void decode_balanced_merge_kernel(const int32_t *__restrict__ sel_count, int hkv,
                                                                   int max_sel, const float *__restrict__ part_o,
                                                                   const float *__restrict__ part_ml,
                                                                   float *__restrict__ out, int hq) {
    constexpr int VD = D / 64, SB = 8;
    args_ready(sel_count, hkv, max_sel, part_o, part_ml, out, hq);
    const int j = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int rows = (int)gridDim.y * hkv, g = hq / hkv;
    const int r = b * hkv + j / g, jj = j - (j / g) * g;
    int all = 0, before = 0, nr = 0;
    for (int k = lane; k < rows; k += 64) {
        const int c = bal_count(sel_count, k, max_sel);
        all += c;
        before += k < r ? c : 0;
        nr += k == r ? c : 0;
    }
    all = wave_isum_all(all);
    before = wave_isum_all(before);
    nr = wave_isum_all(nr);
    const int qn = bal_quantum(all);
    const int w0 = before / qn;
    const int nseg = nr > 0 ? (before + nr - 1) / qn - w0 + 1 : 0;
    const int64_t prow0 = (int64_t)(r + w0) * g + jj;  // segment k: partial row prow0 + k g
    float M = -INFINITY;
    for (int k = lane; k < nseg; k += 64) M = fmaxf(M, part_ml[(prow0 + (int64_t)k * g) * 2]);
    M = wave_max_all(M);
    float acc[VD], lw = 0.f;
#pragma unroll
    for (int dd = 0; dd < VD; ++dd) acc[dd] = 0.f;
    for (int k0 = 0; k0 < nseg; k0 += 64) {
        const int kn = min(64, nseg - k0);
        float2 ml = make_float2(-INFINITY, 0.f);
        if (lane < kn) ml = *reinterpret_cast<const float2 *>(part_ml + (prow0 + (int64_t)(k0 + lane) * g) * 2);
        const float f = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
        lw += wave_sum_all(f * ml.y);
        for (int i0 = 0; i0 < kn; i0 += SB) {
            float ov[SB][VD];
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                const float *p = part_o + (prow0 + (int64_t)(k0 + min(i0 + i, kn - 1)) * g) * D + VD * lane;
                if constexpr (VD == 2) {
                    const float2 x = *reinterpret_cast<const float2 *>(p);
                    ov[i][0] = x.x, ov[i][1] = x.y;
                } else {
                    ov[i][0] = p[0];
                }
            }
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), min(i0 + i, 63)));
                const bool use = i0 + i < kn;
#pragma unroll
                for (int dd = 0; dd < VD; ++dd) acc[dd] = use ? fmaf(ws, ov[i][dd], acc[dd]) : acc[dd];
            }
        }
    }
    const int64_t row = (int64_t)b * hq + j;
    const float inv = 1.0f / lw;
    if constexpr (VD == 2) {
        reinterpret_cast<float2 *>(out + row * D)[lane] = make_float2(acc[0] * inv, acc[1] * inv);
    } else {
        out[row * D + lane] = acc[0] * inv;
    }
}

// Merge of the splits of one (sequence, query head) per wave (the arithmetic
// is merge_split_row in decode_common.h).
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(int splits, const float *__restrict__ part_o,
                                                          const float *__restrict__ part_ml, float *__restrict__ out,
                                                          int hq) {
    args_ready(splits, part_o, part_ml, hq);
    const int j = blockIdx.x, b = blockIdx.y;
    merge_split_row<D>(splits, part_o, part_ml, out, (int64_t)b * hq + j, threadIdx.x);
}

template <typename T, int D, int GP>
static void launch_decode_t(const void *q, int hq, const KvView &kv, const ChunkView &ch, const int32_t *sel_idx,
                            const int32_t *sel_count, int max_sel, float scale_log2, int splits, float *out,
                            float *part_o, float *part_ml, hipStream_t s) {
    dim3 grid(splits, kv.hkv, kv.batch), block(kDecWaves * 64);
    const int max_items = sel_idx ? max_sel : ch.max_chunks;
    if (!ch.starts && kv.page == 16)
        hipLaunchKernelGGL((decode_paged16_kernel<T, D, GP, BSA_DECODE_PD>), grid, block, 0, s, (const T *)q, hq, kv, sel_idx,
                           sel_count, max_sel, scale_log2, splits, out, part_o, part_ml);
    else if (kv.page >= 16 && max_items <= kSegItems)
        hipLaunchKernelGGL((decode_segments_kernel<T, D, GP>), grid, block, 0, s, (const T *)q, hq, kv, ch, sel_idx,
                           sel_count, max_sel, scale_log2, splits, out, part_o, part_ml);
    else
        hipLaunchKernelGGL((decode_chunked_kernel<T, D, GP>), grid, block, 0, s, (const T *)q, hq, kv, ch, sel_idx,
                           sel_count, max_sel, scale_log2, splits, out, part_o, part_ml);
}

template <typename T, int D>
static void launch_decode_g(const void *q, int hq, const KvView &kv, const ChunkView &ch, const int32_t *sel_idx,
                            const int32_t *sel_count, int max_sel, float scale_log2, int splits, float *out,
                            float *part_o, float *part_ml, hipStream_t s) {
    const int g = hq / kv.hkv;
    if (g <= 4)
        launch_decode_t<T, D, 4>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o, part_ml,
                                 s);
    else if (g <= 8)
        launch_decode_t<T, D, 8>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o, part_ml,
                                 s);
    else
        launch_decode_t<T, D, 16>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                  part_ml, s);
}

hipError_t launch_decode(const void *q, int32_t hq, const KvView &kv, const ChunkView &ch, const int32_t *sel_idx,
                         const int32_t *sel_count, int32_t max_sel, float scale, int32_t splits, float *out, void *ws,
                         hipStream_t s) {
    const float scale_log2 = scale * kLog2e;
    float *part_o = nullptr, *part_ml = nullptr;
    if (splits > 1) {
        part_o = (float *)ws;
        part_ml = part_o + (size_t)kv.batch * hq * splits * kv.d;
    }
    if (kv.dtype == BSA_BF16) {
        if (kv.d == 128)
            launch_decode_g<uint16_t, 128>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                           part_ml, s);
        else
            launch_decode_g<uint16_t, 64>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                          part_ml, s);
    } else {
        if (kv.d == 128)
            launch_decode_g<float, 128>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                        part_ml, s);
        else
            launch_decode_g<float, 64>(q, hq, kv, ch, sel_idx, sel_count, max_sel, scale_log2, splits, out, part_o,
                                       part_ml, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1 || !out) return e;  // no out: the partials are the result
    return launch_decode_merge(splits, part_o, part_ml, out, hq, kv.batch, kv.d, s);
}

template <typename T, int D, int GP>
static void launch_balanced_t(const void *q, int hq, const KvView &kv, const int32_t *sel_idx,
                              const int32_t *sel_count, int max_sel, float scale_log2, float *part_o, float *part_ml,
                              hipStream_t s) {
    hipLaunchKernelGGL((decode_balanced_kernel<T, D, GP, BSA_DECODE_PD>), dim3(kBalWgs), dim3(kDecWaves * 64), 0, s,
                       (const T *)q, hq, kv, sel_idx, sel_count, max_sel, scale_log2, part_o, part_ml);
}

template <typename T, int D>
static void launch_balanced_g(const void *q, int hq, const KvView &kv, const int32_t *sel_idx,
                              const int32_t *sel_count, int max_sel, float scale_log2, float *part_o, float *part_ml,
                              hipStream_t s) {
    const int g = hq / kv.hkv;
    if (g <= 4)
        launch_balanced_t<T, D, 4>(q, hq, kv, sel_idx, sel_count, max_sel, scale_log2, part_o, part_ml, s);
    else if (g <= 8)
        launch_balanced_t<T, D, 8>(q, hq, kv, sel_idx, sel_count, max_sel, scale_log2, part_o, part_ml, s);
    else
        launch_balanced_t<T, D, 16>(q, hq, kv, sel_idx, sel_count, max_sel, scale_log2, part_o, part_ml, s);
}

hipError_t launch_decode_balanced(const void *q, int32_t hq, const KvView &kv, const int32_t *sel_idx,
                                  const int32_t *sel_count, int32_t max_sel, float scale, float *out, void *ws,
                                  hipStream_t s) {
    const float scale_log2 = scale * kLog2e;
    const int g = hq / kv.hkv;
    float *part_o = (float *)ws;
    float *part_ml = part_o + (size_t)(kv.batch * kv.hkv + kBalWgs) * g * kv.d;
    if (kv.dtype == BSA_BF16) {
        if (kv.d == 128)
            launch_balanced_g<uint16_t, 128>(q, hq, kv, sel_idx, sel_count, max_sel, scale_log2, part_o, part_ml, s);
        else
            launch_balanced_g<uint16_t, 64>(q, hq, kv, sel_idx, sel_count, max_sel, scale_log2, part_o, part_ml, s);
    } else {
        if (kv.d == 128)
            launch_balanced_g<float, 128>(q, hq, kv, sel_idx, sel_count, max_sel, scale_log2, part_o, part_ml, s);
        else
            launch_balanced_g<float, 64>(q, hq, kv, sel_idx, sel_count, max_sel, scale_log2, part_o, part_ml, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid(hq, kv.batch);
    if (kv.d == 128)
        hipLaunchKernelGGL(decode_balanced_merge_kernel<128>, grid, dim3(64), 0, s, sel_count, kv.hkv, max_sel, part_o,
                           part_ml, out, hq);
    else
        hipLaunchKernelGGL(decode_balanced_merge_kernel<64>, grid, dim3(64), 0, s, sel_count, kv.hkv, max_sel, part_o,
                           part_ml, out, hq);
    return hipGetLastError();
}

hipError_t launch_decode_merge(int splits, const float *part_o, const float *part_ml, float *out, int hq, int batch,
                               int d, hipStream_t s) {
    dim3 grid(hq, batch);
    if (d == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(64), 0, s, splits, part_o, part_ml, out, hq);
    else
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(64), 0, s, splits, part_o, part_ml, out, hq);
    return hipGetLastError();
}

}  // namespace bsa
