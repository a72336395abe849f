// ceiling.hip -- the read-bandwidth ceiling of the sparse decode's access
// pattern, for the benchmark only (libbsa_ceiling.so; nothing on the
// attention path calls it).
//
// A decode launch streams the selected pages of every (sequence, KV head) row:
// K and V runs of 4 KiB each (16 tokens x 128 dims x 2 bytes) at scattered
// addresses.  This kernel reads the same kind of runs with none of the
// attention's arithmetic: each wave takes `per_wave` consecutive entries of a
// run list, keeps four runs (16 KiB) in flight, and folds the words into a
// checksum whose store never fires.  Timed on a fresh random run list per
// launch, it tells what any kernel moving the same bytes in one launch can
// reach on this part (ramp-up and tail included).
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

constexpr int kRunWords = 4096 / 16;   // 16-byte words per 4 KiB run
constexpr int kInFlight = 4;           // runs in flight per wave

__global__ __launch_bounds__(256) void gather_runs_kernel(const uint4 *__restrict__ base,
                                                          const int32_t *__restrict__ runs, int32_t n_runs,
                                                          int32_t per_wave, uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t first = wave * per_wave;
    const int32_t count = (int32_t)min((int64_t)per_wave, max((int64_t)0, (int64_t)n_runs - first));
    if (count == 0) return;
    const int32_t *my = runs + first;
    uint32_t acc = 0;
    uint4 buf[kInFlight][4];
#pragma unroll
    for (int f = 0; f < kInFlight; ++f) {
        const uint4 *r = base + (int64_t)my[min(f, count - 1)] * kRunWords;
#pragma unroll
        for (int j = 0; j < 4; ++j) buf[f][j] = r[lane + 64 * j];
    }
    for (int i = 0; i < count; i += kInFlight) {
#pragma unroll
        for (int f = 0; f < kInFlight; ++f) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc ^= buf[f][j].x ^ buf[f][j].y ^ buf[f][j].z ^ buf[f][j].w;
            // the next run of this slot, clamped to the last one of the list
            // (a repeated run is an L2 hit, not HBM traffic)
            const uint4 *r = base + (int64_t)my[min(i + kInFlight + f, count - 1)] * kRunWords;
#pragma unroll
            for (int j = 0; j < 4; ++j) buf[f][j] = r[lane + 64 * j];
        }
    }
#pragma unroll
    for (int f = 0; f < kInFlight; ++f)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc ^= buf[f][j].x ^ buf[f][j].y ^ buf[f][j].z ^ buf[f][j].w;
    if (acc == 0x9e3779b9u) sink[0] = acc;   // keeps the loads; practically never taken
}

}  // namespace

// Reads runs[0 .. n_runs) (4 KiB run indices into `base`, each in
// [0, buffer bytes / 4096): the caller guarantees it) with per_wave runs per
// wave and 4 waves per workgroup.  Returns a hipError_t value (0 = launched).
extern "C" int bsa_ceiling_gather(const void *base, const int32_t *runs, int32_t n_runs, int32_t per_wave,
                                  uint32_t *sink, void *stream) {
    if (!base || !runs || !sink || n_runs < 1 || per_wave < 1) return (int)hipErrorInvalidValue;
    const int64_t waves = ((int64_t)n_runs + per_wave - 1) / per_wave;
    const int64_t grid = (waves + 3) / 4;
    if (grid > 0x7fffffff) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(gather_runs_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)base, runs, n_runs, per_wave, sink);
    return (int)hipGetLastError();
}
