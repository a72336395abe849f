// tile_prefill.hip -- causal prefill attention of query tiles over their
// selected key blocks, on the matrix cores.
//
// Source: "Technische Samenvatting: Onzekerheidsgestuurde Selectie voor
// Blok-schaarse Aandacht", section "Methodologie" step 5: every tile attends to
// the blocks of its (sentinel-padded) kv_idx row; padding keeps one dispatch
// shape for expanded and base tiles, and the kernel stops at the first
// sentinel, so an untriggered tile costs its k blocks only.
//
// One workgroup per (tile, KV head, row half): one wave per query head of the
// GQA group, 32 rows per wave (two 16-row MFMA column tiles), so each staged
// K/V block feeds G x 32 query rows.  Per selected 64-key block:
//   S^T[key][row] = K . Q^T      16 v_mfma_f32_16x16x32_bf16 per row tile,
//                                Q^T in VGPRs, K rows read from LDS in a
//                                permuted order (below)
//   online softmax once per block per row (fp32, log2 domain); the row is the
//   MFMA column, so its 16 keys per lane reduce with two cross-lane maxes
//   O^T[dim][row] += V^T . P^T   16 v_mfma_f32_16x16x32_f16 per row tile
// K tile kt (16 keys) of 32-key chunk c holds, in MFMA row 4a + i, the key
// 32c + 8a + 4(kt & 1) + i.  The S^T accumulator of lane (row, a) then holds
// keys 32c + 8a .. 32c + 8a + 7 across the chunk's two tiles, which is exactly
// the 8-key slice of P^T that lane supplies to the P.V product.
//
// Staging: K and V blocks are copied straight from global memory into LDS
// (global_load_lds, 16 bytes a lane, 1 KiB = 4 rows of 256 bytes per wave
// instruction), three blocks deep, so no staging registers are needed and
// block b+2 is in flight while block b is computed.  Inside a row the 16-byte
// chunk c is stored at position c ^ swz(row), swz a bijection of row bits
// 0, 1, 3 and 4 (a 256-byte row spans the 64 LDS banks once).  A K operand read
// touches 16 rows (those four bits) at one chunk, so its 16 lanes land on 16
// different positions.  A transposed V read makes each half-wave touch 8 rows
// (bits 0, 1 and 3, or 0, 1 and 4 with 3 fixed) at one 32-byte chunk pair; swz
// bits 1-3 are row bits 0, 1 and (3 xor 4), so those 8 pieces fill the 8 pair
// positions of the bank line.  V arrives already in fp16: a first kernel
// converts the whole V cache once (bf16 -> fp16, into the caller's workspace),
// instead of every workgroup converting each staged block again.  The V^T
// operand (8 keys of one dim per lane) comes from row-major V with two
// ds_read_b64_tr_b16 (4 keys each).
// P is rounded to fp16 and the row sums are taken from the rounded values on
// the matrix cores (an all-ones A operand); bf16 -> fp16 is exact for |v| in
// the fp16 normal range.  Keys after a row are masked
// only in the diagonal block.
#include "lds_dma.h"

namespace bsa {

constexpr int kPfD = 128;
constexpr int kPfBlock = 64;
constexpr int kPfRowsPerWave = 32;
constexpr int kPfRowBytes = kPfD * 2;                 // 256 bytes per staged row
constexpr int kPfBlockBytes = kPfBlock * kPfRowBytes;  // 16 KiB for K or V
constexpr int kPfStageBytes = 2 * kPfBlockBytes;       // K then V
constexpr int kPfStages = 3;
constexpr int kPfMaxList = 1024;                       // selected blocks per (tile, KV head) held in LDS
constexpr int kPfInstrs = kPfStageBytes / 1024;        // 1 KiB wave instructions per block

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_raw __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_raw lds_f16x4_t;

__device__ __forceinline__ int pf_swz(int row) {
    return ((row >> 4) & 1) | ((row & 3) << 1) | ((((row >> 3) ^ (row >> 4)) & 1) << 3);
}

// Issue this wave's share of one block's copy into stage `buf` (lds byte
// address): wave instruction u (u < 16: K rows 4u..4u+3, else V rows), lane
// l writes row 4(u mod 16) + l/16 at chunk position l mod 16, so it loads
// chunk (l mod 16) ^ swz(row).  Every wave issues the same count.  The cache
// is token-major: token pos of a head starts at base + pos * row_bytes.
// A block inside the sequence is copied from a wave-uniform block base plus
// the lane offsets of `coff` (fixed per wave and instruction); the ragged last
// block clamps rows past the end onto the last row (those keys are masked).
template <int G>
__device__ __forceinline__ void issue_block(char *lds_stage, const uint16_t *kbase, const uint16_t *vbase,
                                            int64_t krow_bytes, int64_t vrow_bytes, const uint32_t *coff, int blk,
                                            int rows, int w, int lane) {
    constexpr int NI = (kPfInstrs + G - 1) / G;
    if ((blk + 1) * kPfBlock <= rows) {
        const char *kb = reinterpret_cast<const char *>(kbase) + (int64_t)blk * kPfBlock * krow_bytes;
        const char *vb = reinterpret_cast<const char *>(vbase) + (int64_t)blk * kPfBlock * vrow_bytes;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int u = min(w + G * i, kPfInstrs - 1);  // duplicates rewrite identical bytes
            dma16_sbase(u < 16 ? kb : vb, coff[i], lds_addr(lds_stage) + u * 1024);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int u = min(w + G * i, kPfInstrs - 1);
        const int row = 4 * (u & 15) + (lane >> 4);
        const int chunk = (lane & 15) ^ pf_swz(row);
        const int pos = min(blk * kPfBlock + row, rows - 1);
        const char *src = u < 16 ? reinterpret_cast<const char *>(kbase) + pos * krow_bytes + chunk * 16
                                 : reinterpret_cast<const char *>(vbase) + pos * vrow_bytes + chunk * 16;
        dma16(src, lds_addr(lds_stage) + u * 1024);
    }
}

template <int G>
__global__ __launch_bounds__(64 * G) void tile_prefill_kernel(const uint16_t *__restrict__ q, int hq, int rows,
                                                              KvView kv, const uint16_t *__restrict__ v16,
                                                              const int32_t *__restrict__ kv_idx,
                                                              int idx_stride, float scale_log2,
                                                              float *__restrict__ out) {
    constexpr int NT = 64 * G;
    constexpr int NI = (kPfInstrs + G - 1) / G;
    // three distinct LDS objects (not one array): each unrolled step names its
    // buffers statically, so the compiler can tell that the copy in flight
    // never aliases the buffer being read and adds no wait for it
    __shared__ __attribute__((aligned(1024))) char stage0[kPfStageBytes];
    __shared__ __attribute__((aligned(1024))) char stage1[kPfStageBytes];
    __shared__ __attribute__((aligned(1024))) char stage2[kPfStageBytes];
    __shared__ int blist[kPfMaxList];
    __shared__ int nblk_s;
    // Tiles in descending order: causal tiles with the most blocks start first.
    // The two row halves of a tile copy the same blocks, so they take
    // workgroups 8 apart: the dispatcher deals workgroups to the 8 XCDs
    // round-robin, which puts both halves on one XCD, and the second half's
    // copies hit that XCD's L2.  Groups of 16 workgroups hold both halves of 8
    // consecutive tiles (the last group those of the remaining tiles).
    const int n_tiles = gridDim.x >> 1, grp = blockIdx.x >> 4, pos = blockIdx.x & 15;
    const int in_grp = min(8, n_tiles - 8 * grp);
    const int t = n_tiles - 1 - (8 * grp + pos % in_grp), half = pos / in_grp, h = blockIdx.y;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n16 = lane & 15, G4 = lane >> 4;
    const int j = h * G + w;
    const int rbase = t * kPfBlock + half * kPfRowsPerWave;
    const uint16_t *kbase = reinterpret_cast<const uint16_t *>(kv.k) + (int64_t)h * kv.sh;
    const uint16_t *vbase = v16 + (int64_t)h * kPfD;                 // fp16 V [rows][H_kv][D]
    const int64_t row_bytes = kv.st * 2;  // token-major: stride_page == 64 * stride_token (host-checked)
    const int64_t vrow_bytes = (int64_t)kv.hkv * kPfD * 2;

    // the visible selected blocks: a prefix of the ascending, -1 padded row
    // (idx_stride <= kPfMaxList, host-checked); dense: blocks 0 .. t
    const int32_t *idx = kv_idx ? kv_idx + ((int64_t)t * kv.hkv + h) * idx_stride : nullptr;
    if (threadIdx.x == 0) nblk_s = idx ? idx_stride : t + 1;
    __syncthreads();
    if (idx) {
        for (int i = threadIdx.x; i < idx_stride; i += NT) {
            const int blk = idx[i];
            blist[i] = blk;
            if (blk < 0 || blk > t) atomicMin(&nblk_s, i);
        }
    }
    // Q^T operand: rows rbase + 16*rt + n16, dims 32s + 8*G4 .. +8
    bf16x8 qb[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = min(rbase + 16 * rt + n16, rows - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qb[rt][s] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(q + ((int64_t)r * hq + j) * kPfD + 32 * s + 8 * G4));
    }
    f32x4 o[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};
    f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const f16x8 ones = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                        (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
    __syncthreads();
    const int nb = nblk_s;
    auto block_at = [&](int i) {
        return __builtin_amdgcn_readfirstlane(idx ? blist[min(i, max(nb - 1, 0))] : min(i, t));
    };
    // lane byte offsets of this wave's copy instructions inside a block
    // (64 rows of either cache fit in 32 bits: host-checked)
    uint32_t coff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int u = min(w + G * i, kPfInstrs - 1);
        const int row = 4 * (u & 15) + (lane >> 4);
        const int chunk = (lane & 15) ^ pf_swz(row);
        coff[i] = (uint32_t)(row * (u < 16 ? row_bytes : vrow_bytes) + chunk * 16);
    }

    // prologue: blocks 0 and 1 copied.  Everything this wave loaded so far (Q
    // included) is waited for here, so the compiler, which does not see the
    // copies, needs no wait of its own in the loop.
    if (nb > 0) {
        issue_block<G>(stage0, kbase, vbase, row_bytes, vrow_bytes, coff, block_at(0), rows, w, lane);
        issue_block<G>(stage1, kbase, vbase, row_bytes, vrow_bytes, coff, block_at(1), rows, w, lane);
    }
    wait_vmcnt<0>();
    wait_lgkm0();
    stage_barrier();
    // Per-lane LDS byte offsets, the same for every block.  The K row of MFMA
    // row n16 in tile kt is 32(kt>>1) + 4(kt&1) + krow_lo and the V rows read
    // by lane (n16, G4) are 32c + 8G4 + 4hh + (n16>>2): the swizzle ignores
    // row bits 2 and 5, so it is that of krow_lo, or of 8G4 + (n16>>2),
    // whatever kt, c and hh are.  The lane's 8-byte piece of V dims
    // 16dt + 4(n16&3) is chunk 2dt + ((n16>>1)&1), half n16&1.
    const int krow_lo = 8 * (n16 >> 2) + (n16 & 3);
    int koff[4], voff[8];
#pragma unroll
    for (int st = 0; st < 4; ++st) koff[st] = krow_lo * kPfRowBytes + 16 * ((4 * st + G4) ^ pf_swz(krow_lo));
    {
        const int vrow = 8 * G4 + (n16 >> 2);
        const int vswz = pf_swz(vrow);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            voff[dt] = vrow * kPfRowBytes + 16 * ((2 * dt + ((n16 >> 1) & 1)) ^ vswz) + 8 * (n16 & 1);
    }
    // one block: bcur holds block ii, bn1 receives block ii+1 (in flight), bn2
    // block ii+2 (issued here; last read a block ago, before the barrier)
    auto step = [&](int ii, char *bcur, char *bn1, char *bn2) {
        const int blk = block_at(ii);
        issue_block<G>(bn2, kbase, vbase, row_bytes, vrow_bytes, coff, block_at(ii + 2), rows, w, lane);
        const char *kc = bcur;
        const char *vc = bcur + kPfBlockBytes;
        const bool diag = blk == t;
        // S^T for the 64 keys: 4 key tiles x 2 row tiles
        // feature steps outermost, so the 8 accumulators of a step are
        // independent MFMA chains; each step's 4 K operands are read one step
        // ahead (measured 3 % faster than key tiles outermost with the reads
        // next to their use; two steps ahead, or also reading V ahead, gained
        // nothing).  Every accumulator still sums its steps in the same order.
        f32x4 s[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) s[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto kread = [&](int kt, int st) {
            const int key0 = 32 * (kt >> 1) + 4 * (kt & 1);  // + krow_lo (in koff)
            return *reinterpret_cast<const bf16x8 *>(kc + key0 * kPfRowBytes + koff[st]);
        };
        bf16x8 ka[2][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) ka[0][kt] = kread(kt, 0);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (st + 1 < 4) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) ka[(st + 1) & 1][kt] = kread(kt, st + 1);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the next step's reads ahead of these MFMAs
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    s[kt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[st & 1][kt], qb[rt][st], s[kt][rt], 0, 0, 0);
        }
        // online softmax, one step per block and row.  Masks only where a key
        // can be invisible (the diagonal block, the ragged last block); the
        // scale is folded into the exponent's FMA (max taken on raw scores,
        // the scale being positive).
        const bool need_mask = diag || (blk + 1) * kPfBlock > rows;
        f16x8 pb[2][2];  // [key chunk][row tile]
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (need_mask) {
                const int r = rbase + 16 * rt + n16;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int pos = blk * kPfBlock + 32 * (kt >> 1) + 8 * G4 + 4 * (kt & 1) + i;
                        if (!(pos < rows && (!diag || pos <= r))) s[kt][rt][i] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kt][rt][i]);
            mx = max_across_rows16(mx);
            // Lazy rescale: the reference max moves only when a row's max
            // exceeds it by more than 2^8 (weights stay <= 256, well inside
            // fp16), so most blocks skip rescaling the accumulators; the sums
            // use the same reference, so the result is exact.
            const float mb = mx * scale_log2;
            const bool grow = mb > m_run[rt] + 8.f;
            if (__ballot(grow)) {
                const float m_new = grow ? mb : m_run[rt];
                const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_new);  // 0 from -inf
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[dt][rt] *= alpha;
                lsum[rt] *= alpha;
                m_run[rt] = m_new;
            }
            const float m_use = m_run[rt] == -INFINITY ? 0.f : m_run[rt];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pb[kt >> 1][rt][4 * (kt & 1) + i] =
                        (_Float16)__builtin_amdgcn_exp2f(fmaf(s[kt][rt][i], scale_log2, -m_use));
        }
        // O^T += V^T . P^T over the two 32-key chunks: lane (dim 16dt + n16, G4)
        // supplies keys 32c + 8*G4 .. +7, read as two transposed 4-key pieces
        // (lane L of the 16-lane group points at row rb + L/4, dims 16dt + 4(L%4))
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                f16x4 pr[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const char *p = vc + (32 * c + 4 * hh) * kPfRowBytes + voff[dt];
                    pr[hh] = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4_t *)p));
                }
                const f16x8 a = {pr[0][0], pr[0][1], pr[0][2], pr[0][3], pr[1][0], pr[1][1], pr[1][2], pr[1][3]};
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[c][rt], o[dt][rt], 0, 0, 0);
            }
            // row sums of the rounded weights: an all-ones A operand (every
            // output row of this tile is the column sum of P^T)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[c][rt], lsum[rt], 0, 0, 0);
        }
        // block ii+1 has landed (only block ii+2's copies may be outstanding)
        // and this wave's reads of bcur are done
        (void)bn1;
        wait_vmcnt<NI>();
        wait_lgkm0();
        stage_barrier();
    };
    for (int ii = 0; ii < nb; ii += 3) {
        step(ii, stage0, stage1, stage2);
        if (ii + 1 < nb) step(ii + 1, stage1, stage2, stage0);
        if (ii + 2 < nb) step(ii + 2, stage2, stage0, stage1);
    }
    wait_vmcnt<0>();  // this wave's copies have landed
    stage_barrier();  // and every other wave's: the ring is free
    // Normalise and write.  Lane (n16, G4) holds O^T[dim 16dt + 4*G4 + i][row
    // 16rt + n16]: written straight out, each store would cover 64 bytes of 16
    // rows.  Staged per row tile through this wave's corner of the ring (16
    // rows, padded stride), each store covers two whole 512-byte rows instead
    // (measured 2 % faster at 131,072 tokens; the output is 1.9 GB of fp32).
    {
        constexpr int RS = kPfD + 4;  // floats per staged row
        static_assert(3 * 16 * RS * 4 <= kPfStageBytes, "three waves' rows per stage");
        float *stg = reinterpret_cast<float *>(w < 3 ? stage0 : (w < 6 ? stage1 : stage2)) + (w % 3) * (16 * RS);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const float inv = 1.0f / lsum[rt][0];  // every row of the sum tile holds the row's total
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const f32x4 v = o[dt][rt] * inv;
                *reinterpret_cast<float4 *>(stg + n16 * RS + 16 * dt + 4 * G4) = make_float4(v[0], v[1], v[2], v[3]);
            }
            // (a wave's LDS accesses run in order: these reads see the writes
            // above, and the next row tile's writes follow these reads)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = 2 * i + (lane >> 5), col = (lane & 31) * 4;
                const float4 x = *reinterpret_cast<const float4 *>(stg + row * RS + col);
                const int r = rbase + 16 * rt + row;
                if (r < rows) *reinterpret_cast<float4 *>(out + ((int64_t)r * hq + j) * kPfD + col) = x;
            }
        }
    }
}

// V (bf16, cache strides) -> fp16 [rows][H_kv][D], 8 values per thread,
// rounded to nearest even.
__global__ __launch_bounds__(256) void v_to_fp16_kernel(KvView kv, int rows, uint16_t *__restrict__ v16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte piece
    const int per_row = kv.hkv * (kPfD / 8);
    if (i >= (int64_t)rows * per_row) return;
    const int r = (int)(i / per_row), rem = (int)(i % per_row), h = rem / (kPfD / 8), d = (rem % (kPfD / 8)) * 8;
    const uint4 x = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(kv.v) + r * kv.st +
                                                     h * kv.sh + d);
    const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
    uint32_t y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const _Float16 lo = (_Float16)bf16_lo(wd[e]), hi = (_Float16)bf16_hi(wd[e]);
        y[e] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    *reinterpret_cast<uint4 *>(v16 + (int64_t)(r * kv.hkv + h) * kPfD + d) = make_uint4(y[0], y[1], y[2], y[3]);
}

hipError_t launch_tile_prefill(const void *q, int32_t hq, int32_t rows, const KvView &kv, int32_t tile_rows,
                               const int32_t *kv_idx, int32_t idx_stride, float scale, float *out, void *ws,
                               hipStream_t s) {
    (void)tile_rows;  // validated: == 64 == kv.page
    uint16_t *v16 = (uint16_t *)ws;
    const int64_t pieces = (int64_t)rows * kv.hkv * (kPfD / 8);
    hipLaunchKernelGGL(v_to_fp16_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, kv, rows, v16);
    const int g = hq / kv.hkv;
    const int n_tiles = (rows + kPfBlock - 1) / kPfBlock;
    dim3 grid(n_tiles * 2, kv.hkv), block(64 * g);
    const float sl = scale * kLog2e;
#define BSA_TP(G)                                                                                            \
    case G:                                                                                                  \
        hipLaunchKernelGGL(tile_prefill_kernel<G>, grid, block, 0, s, (const uint16_t *)q, hq, rows, kv, v16,    \
                           kv_idx, idx_stride, sl, out);                                                     \
        break;
    switch (g) {
        BSA_TP(1) BSA_TP(2) BSA_TP(3) BSA_TP(4) BSA_TP(5) BSA_TP(6) BSA_TP(7) BSA_TP(8)
    default:
        return hipErrorInvalidValue;
    }
#undef BSA_TP
    return hipGetLastError();
}

}  // namespace bsa
