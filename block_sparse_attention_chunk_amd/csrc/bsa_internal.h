// bsa_internal.h -- device helpers and launcher declarations shared by the
// libbsa HIP sources (gfx950 only).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsa.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 <-> f32 on raw bits ------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
// exact for values that are already representable in bf16 (min / max of bf16s)
__device__ __forceinline__ uint16_t f32_to_bf16_exact(float x) { return uint16_t(__float_as_uint(x) >> 16); }
// round to nearest even (finite values)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    return uint16_t((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---- order-preserving float keys --------------------------------------------
// key(a) < key(b)  <=>  a < b  for non-NaN floats (-0 sorts below +0).
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// ---- wave-level helpers (wave64) --------------------------------------------

// Max over lanes l, l^16, l^32, l^48 (the same position in the wave's four
// 16-lane rows) with the gfx950 row-swap instructions: permlane16_swap of a
// register with itself yields (v[l], v[l^16]) and permlane32_swap yields
// (v[l], v[l^32]) in every lane; no LDS round trip.
__device__ __forceinline__ float max_across_rows16(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}

// Sum over lanes l, l^16, l^32, l^48, the same way.
__device__ __forceinline__ float sum_across_rows16(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    v = __int_as_float(a[0]) + __int_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

// Maximum and sum over all 64 lanes of a wave, in every lane: DPP shifts
// inside each 16-lane row, then rows combined (lane 63 ends with the total),
// broadcast with readlane.  No LDS round trip.
#define BSA_DPP_F(x, ctrl, rmask, ident) \
    __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(x), ctrl, rmask, 0xf, false))
__device__ __forceinline__ float wave_max_all(float x) {
    x = fmaxf(x, BSA_DPP_F(x, 0x111, 0xf, -INFINITY));  // row_shr:1
    x = fmaxf(x, BSA_DPP_F(x, 0x112, 0xf, -INFINITY));  // row_shr:2
    x = fmaxf(x, BSA_DPP_F(x, 0x114, 0xf, -INFINITY));  // row_shr:4
    x = fmaxf(x, BSA_DPP_F(x, 0x118, 0xf, -INFINITY));  // row_shr:8
    x = fmaxf(x, BSA_DPP_F(x, 0x142, 0xa, -INFINITY));  // row_bcast:15
    x = fmaxf(x, BSA_DPP_F(x, 0x143, 0xc, -INFINITY));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_sum_all(float x) {
    x += BSA_DPP_F(x, 0x111, 0xf, 0.f);
    x += BSA_DPP_F(x, 0x112, 0xf, 0.f);
    x += BSA_DPP_F(x, 0x114, 0xf, 0.f);
    x += BSA_DPP_F(x, 0x118, 0xf, 0.f);
    x += BSA_DPP_F(x, 0x142, 0xa, 0.f);
    x += BSA_DPP_F(x, 0x143, 0xc, 0.f);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
#undef BSA_DPP_F

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- kernel arguments ----------------------------------------------------------
// Arguments reach the scalar registers by scalar loads that the compiler emits
// at first use; spread over a kernel's prologue they form a chain of dependent
// round trips ahead of the first memory requests.  Naming the arguments the
// first requests need here makes the compiler fetch them together, with a
// single wait.
template <typename A>
__device__ __forceinline__ void arg_ready(const A &a) {
    asm volatile("" ::"s"(a));
}
template <typename... A>
__device__ __forceinline__ void args_ready(const A &...a) {
    (arg_ready(a), ...);
}

// ---- launchers (defined in the .hip files) -----------------------------------
struct KvView {
    const void *k, *v;
    int64_t sp, sh, st;
    const int32_t *bt;
    const int32_t *seq_lens;
    int32_t batch, hkv, d, page, log2page, max_pages, dtype;
};

struct ChunkView {
    const int32_t *starts;   // NULL = fixed pages
    const int32_t *num;
    int32_t max_chunks;
};

hipError_t launch_chunk_meta(const KvView &kv, const ChunkView &ch, void *kmin, void *kmax, float *cen,
                             uint32_t which, const int32_t *from_len, int32_t max_touched, hipStream_t s);
hipError_t launch_score_decode(const void *q, int32_t hq, const KvView &kv, const ChunkView &ch, const void *kmin,
                               const void *kmax, const float *cen, int32_t kind, float *scores, hipStream_t s);
hipError_t launch_score_tiles(const void *q, int32_t hq, int32_t rows, int32_t tile_rows, const KvView &kv,
                              int32_t n_blocks, const void *kmin, const void *kmax, const float *cen, int32_t kind,
                              int32_t causal, float *scores, hipStream_t s);
hipError_t launch_select(const float *scores, const KvView &kv, const ChunkView &ch, const bsa_budget &b,
                         int32_t *sel_idx, int32_t *sel_count, int32_t max_sel, hipStream_t s);
hipError_t launch_router(const float *ts, int32_t n_tiles, int32_t hkv, int32_t n_blocks, int32_t causal, int32_t k,
                         int32_t rho, float quantile, float fixed, int32_t *kv_idx, float *sigma, float *sigma_bar,
                         uint8_t *triggered, float *threshold, void *ws, hipStream_t s);
hipError_t launch_decode(const void *q, int32_t hq, const KvView &kv, const ChunkView &ch, const int32_t *sel_idx,
                         const int32_t *sel_count, int32_t max_sel, float scale, int32_t splits, float *out,
                         void *ws, hipStream_t s);
// Balanced decode schedule (decode.hip): kBalWgs workgroups share the kept
// pages of all rows equally, at least kBalMinItems each; batch x H_kv rows up
// to kBalMaxRows.  Workspace: (rows + kBalWgs) x group entries of (D + 2) floats.
constexpr int kBalWgs = 256;
constexpr int kBalMinItems = 16;
constexpr int kBalMaxRows = 4096;
hipError_t launch_decode_balanced(const void *q, int32_t hq, const KvView &kv, const int32_t *sel_idx,
                                  const int32_t *sel_count, int32_t max_sel, float scale, float *out, void *ws,
                                  hipStream_t s);
hipError_t launch_decode_merge(int splits, const float *part_o, const float *part_ml, float *out, int hq, int batch,
                               int d, hipStream_t s);
hipError_t launch_select_decode(const void *q, int32_t hq, const KvView &kv, const float *scores,
                                const bsa_budget &bud, int32_t *sel_idx, int32_t *sel_count, int32_t max_sel,
                                float scale, int32_t splits, float *out, void *ws, hipStream_t s);
hipError_t launch_tile_prefill(const void *q, int32_t hq, int32_t rows, const KvView &kv, int32_t tile_rows,
                               const int32_t *kv_idx, int32_t idx_stride, float scale, float *out, void *ws,
                               hipStream_t s);

}  // namespace bsa
