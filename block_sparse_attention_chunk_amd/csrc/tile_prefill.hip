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
// GQA group, 32 rows per wave (two 16-row MFMA column tiles).  For each
// selected 64-key block the workgroup stages K (bf16, row-major) and V
// (converted to fp16, transposed to [dim][key]) in LDS once for all heads.
// Per 32-key half:
//   S^T[key][row] = K . Q^T            v_mfma_f32_16x16x32_bf16, Q^T in VGPRs
//   online softmax per row (fp32, log2 domain; the row is the MFMA column, so
//   its 8 keys per lane reduce with two cross-lane maxes)
//   O^T[dim][row] += V^T . P^T         v_mfma_f32_16x16x32_f16
// P^T is built straight from the S^T accumulators of two 16-key tiles; V^T
// uses the same per-lane key order, so the products pair up regardless of
// the instruction's internal k order.  bf16 -> fp16 is exact for |v| in the
// fp16 normal range.  Keys after a row are masked only in the diagonal block.
#include "bsa_internal.h"

namespace bsa {

constexpr int kPfD = 128;
constexpr int kPfBlock = 64;
constexpr int kPfRowsPerWave = 32;
constexpr int kKStride = kPfD + 8;      // bf16 elements per staged K row (+16 B)
constexpr int kVStride = kPfBlock + 8;  // fp16 elements per staged V^T row (+16 B)

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void tile_prefill_kernel(const uint16_t *__restrict__ q, int hq, int rows,
                                                           KvView kv, const int32_t *__restrict__ kv_idx,
                                                           int idx_stride, float scale_log2,
                                                           float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t ks[kPfBlock * kKStride];
    __shared__ __attribute__((aligned(16))) _Float16 vt[kPfD * kVStride];
    const int t = blockIdx.x >> 1, half = blockIdx.x & 1, h = blockIdx.y;
    const int g = hq / kv.hkv;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, G = lane >> 4;
    const int nthreads = blockDim.x;
    const int j = h * g + w;
    const int rbase = t * kPfBlock + half * kPfRowsPerWave;
    const uint16_t *kbase = reinterpret_cast<const uint16_t *>(kv.k) + (int64_t)h * kv.sh;
    const uint16_t *vbase = reinterpret_cast<const uint16_t *>(kv.v) + (int64_t)h * kv.sh;

    // Q^T operand: rows rbase + 16*rt + n16, dims 32s + 8G .. +8
    bf16x8 qb[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = rbase + 16 * rt + n16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r < rows) v = *reinterpret_cast<const uint4 *>(q + ((int64_t)r * hq + j) * kPfD + 32 * s + 8 * G);
            qb[rt][s] = __builtin_bit_cast(bf16x8, v);
        }
    }
    f32x4 o[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    const int32_t *idx = kv_idx ? kv_idx + ((int64_t)t * kv.hkv + h) * idx_stride : nullptr;
    const int nsel = kv_idx ? idx_stride : t + 1;
    for (int ii = 0; ii < nsel; ++ii) {
        const int blk = idx ? idx[ii] : ii;
        if (blk < 0) break;  // sentinels are trailing
        if (blk > t) continue;  // a block after the diagonal holds no visible key
        __syncthreads();     // previous block's LDS reads are done
        // stage K (row-major bf16) and V^T (fp16)
        for (int c = threadIdx.x; c < kPfBlock * (kPfD / 8); c += nthreads) {
            const int key = c >> 4, piece = c & 15;
            const int pos = blk * kPfBlock + key;
            uint4 kw = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
            if (pos < rows) {
                const int64_t off = (int64_t)blk * kv.sp + (int64_t)key * kv.st + piece * 8;
                kw = *reinterpret_cast<const uint4 *>(kbase + off);
                vw = *reinterpret_cast<const uint4 *>(vbase + off);
            }
            *reinterpret_cast<uint4 *>(ks + key * kKStride + piece * 8) = kw;
            const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt[(piece * 8 + 2 * e) * kVStride + key] = (_Float16)bf16_lo(vv[e]);
                vt[(piece * 8 + 2 * e + 1) * kVStride + key] = (_Float16)bf16_hi(vv[e]);
            }
        }
        __syncthreads();
        const bool diag = blk == t;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            f32x4 s[2][2];  // [key tile][row tile]
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) s[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ks + (32 * kh + 16 * kt + n16) * kKStride +
                                                                        32 * st + 8 * G);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
                        s[kt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[rt][st], s[kt][rt], 0, 0, 0);
                }
            }
            f16x8 pb[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int r = rbase + 16 * rt + n16;
                float x[2][4];
                float mx = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int pos = blk * kPfBlock + 32 * kh + 16 * kt + 4 * G + i;
                        const bool ok = pos < rows && (!diag || pos <= r);
                        x[kt][i] = ok ? s[kt][rt][i] * scale_log2 : -INFINITY;
                        mx = fmaxf(mx, x[kt][i]);
                    }
                mx = wave_max_xor(mx, 16);
                mx = wave_max_xor(mx, 32);
                const float m_new = fmaxf(m_run[rt], mx);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = exp2f(m_run[rt] - m_use);
                float psum = 0.f;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const _Float16 p = (_Float16)exp2f(x[kt][i] - m_use);
                        psum += (float)p;  // normalise with the same rounded weights
                        pb[rt][4 * kt + i] = p;
                    }
                l_run[rt] = l_run[rt] * alpha + psum;
                m_run[rt] = m_new;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[dt][rt] *= alpha;
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const _Float16 *vrow = vt + (16 * dt + n16) * kVStride + 32 * kh + 4 * G;
                const f16x4 lo = *reinterpret_cast<const f16x4 *>(vrow);
                const f16x4 hi = *reinterpret_cast<const f16x4 *>(vrow + 16);
                const f16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[rt], o[dt][rt], 0, 0, 0);
            }
        }
    }
    // normalise and write: lane holds O^T[dim 16dt + 4G + i][row 16rt + n16]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        float l = l_run[rt] + __shfl_xor(l_run[rt], 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int r = rbase + 16 * rt + n16;
        if (r < rows) {
            const float inv = 1.0f / l;
            float *orow = out + ((int64_t)r * hq + j) * kPfD;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const f32x4 v = o[dt][rt] * inv;
                *reinterpret_cast<float4 *>(orow + 16 * dt + 4 * G) = make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

hipError_t launch_tile_prefill(const void *q, int32_t hq, int32_t rows, const KvView &kv, int32_t tile_rows,
                               const int32_t *kv_idx, int32_t idx_stride, float scale, float *out, hipStream_t s) {
    (void)tile_rows;  // validated: == 64 == kv.page
    const int g = hq / kv.hkv;
    const int n_tiles = (rows + kPfBlock - 1) / kPfBlock;
    dim3 grid(n_tiles * 2, kv.hkv), block(64 * g);
    hipLaunchKernelGGL(tile_prefill_kernel, grid, block, 0, s, (const uint16_t *)q, hq, rows, kv, kv_idx, idx_stride,
                       scale * kLog2e, out);
    return hipGetLastError();
}

}  // namespace bsa
