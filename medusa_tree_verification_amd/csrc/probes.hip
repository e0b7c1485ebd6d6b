// Peak probes: the two ceilings the verify step's roofline is measured
// against, measured on the device itself (the published MI355X figures are
// 8 TB/s of HBM3E and 2.5 PFLOP/s of dense bf16 MFMA).
//
//  - medusa_probe_read: a linear stream of 16-byte non-temporal loads over a
//    caller buffer, every byte read once, four waves per CU with eight loads
//    (8 KiB of whole 128 B lines per wave) in flight: the fastest read shape
//    measured (plain loads, or sixteen waves per CU, stream about 15% slower);
//    the loaded words are folded into one value per thread so that no load
//    can be dropped.  medusa_probe_read_timed also records each workgroup's
//    start and end on the device's constant-rate clock: workgroups are
//    dispatched round-robin over the XCDs, so workgroup w's share is read by
//    XCD w mod 8, and the stamps show how fast each XCD streams.  Its second
//    pattern reads the buffer as the heads' weight stream does: rows of
//    8 KiB in tiles of 8 rows, each load 8 rows x 128 B (lane l: row
//    (l mod 16) mod 8, 16 B at 64 ((l mod 16) / 8) + 16 (l / 16) of a 128 B
//    step), a wave streaming a contiguous range of tiles in batches of 8
//    steps.
//  - medusa_probe_mfma: independent chains of v_mfma_f32_32x32x16_bf16 on
//    register operands, four waves per CU (one per SIMD, eight accumulator
//    chains each), no memory traffic in the loop.
#include "common.h"
#include "medusa_probes.h"

namespace medusa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeU = 8;          // 16-byte loads in flight per thread
constexpr int kProbeWG = kNumCU;    // one workgroup per CU, each streaming its own share
constexpr int kMfmaWaves = 4;       // one wave per SIMD ...
constexpr int kMfmaChains = 8;      // ... with eight independent accumulator chains

// the 8-row-tile pattern: a wave's share of the workgroup's tiles
__device__ __forceinline__ uint32_t probe_tiles(const char *__restrict__ src, size_t ntile,
                                                uint32_t acc) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int c = lane % 16, g = lane / 16;
    const size_t lo = (size_t)blockIdx.x * ntile / gridDim.x, hi = (size_t)(blockIdx.x + 1) * ntile / gridDim.x;
    const size_t t0 = lo + (hi - lo) * wave / (kProbeThreads / kWave);
    const size_t t1 = lo + (hi - lo) * (wave + 1) / (kProbeThreads / kWave);
    for (size_t t = t0; t < t1; ++t) {
        const char *row = src + (t * 8 + c % 8) * 8192 + 64 * (c / 8) + 16 * g;
        for (int b = 0; b < 8; ++b) {
            u32x4 v[kProbeU];
#pragma unroll
            for (int u = 0; u < kProbeU; ++u) v[u] = ld16_nt(row + b * 1024 + u * 128);
#pragma unroll
            for (int u = 0; u < kProbeU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        }
    }
    return acc;
}

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4 *__restrict__ src,
                                                                   size_t n16, uint32_t *sink,
                                                                   uint32_t *stamps, int pattern) {
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    if (pattern == 1) {   // the same in every thread
        const uint32_t acc = probe_tiles((const char *)src, n16 / 4096, 0u);
        sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
            stamps[2 * blockIdx.x] = (uint32_t)t_start;
            stamps[2 * blockIdx.x + 1] = (uint32_t)t_end;
        }
        return;
    }
    // workgroup w streams its contiguous share; each of a wave's U loads
    // covers one kilobyte
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    uint32_t acc = 0u;
    for (size_t i0 = lo + threadIdx.x; i0 < hi; i0 += (size_t)kProbeThreads * kProbeU) {
        u32x4 v[kProbeU];
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) {
            const size_t i = i0 + (size_t)u * kProbeThreads;
            v[u] = i < hi ? ld16_nt(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
    if (stamps) {   // the same in every thread
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
            stamps[2 * blockIdx.x] = (uint32_t)t_start;
            stamps[2 * blockIdx.x + 1] = (uint32_t)t_end;
        }
    }
}

__global__ __launch_bounds__(kMfmaWaves *kWave) void probe_mfma_kernel(int iters, float *sink) {
    const int lane = threadIdx.x % kWave;
    // operands that the compiler cannot fold: they depend on the lane and
    // on the (uniform) iteration count
    const float seed = (float)(lane + 1) * 1e-3f + (float)iters * 1e-9f;
    u32x4 a, b;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        a[w] = pack_bf16x2(seed * (float)(w + 1), -seed);
        b[w] = pack_bf16x2(seed, seed * (float)(w + 2));
    }
    f32x16 acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c) mma32_step(acc[c], a, b, bf16_t{});
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace medusa

using namespace medusa;

extern "C" size_t medusa_probe_sink_bytes(void) {
    const size_t rd = (size_t)kProbeWG * kProbeThreads * sizeof(uint32_t);
    const size_t mf = (size_t)kNumCU * kMfmaWaves * kWave * sizeof(float);
    return rd > mf ? rd : mf;
}

static int probe_read_launch(const void *buf, size_t bytes, void *sink, uint32_t *stamps,
                             int pattern, void *stream) {
    if (!buf || !sink) return MEDUSA_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0) return MEDUSA_ERR_SHAPE;
    if (pattern == 1 && bytes % (8u * 8192u) != 0) return MEDUSA_ERR_SHAPE;
    hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeWG), dim3(kProbeThreads), 0,
                       (hipStream_t)stream, (const u32x4 *)buf, bytes / 16, (uint32_t *)sink,
                       stamps, pattern);
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
}

extern "C" int medusa_probe_read(const void *buf, size_t bytes, void *sink, void *stream) {
    return probe_read_launch(buf, bytes, sink, nullptr, 0, stream);
}

extern "C" int medusa_probe_read_timed(const void *buf, size_t bytes, void *sink, uint32_t *stamps,
                                       int pattern, void *stream) {
    if (!stamps) return MEDUSA_ERR_NULL;
    if (pattern != 0 && pattern != 1) return MEDUSA_ERR_PARAM;
    return probe_read_launch(buf, bytes, sink, stamps, pattern, stream);
}

extern "C" int medusa_probe_read_workgroups(void) { return kProbeWG; }

extern "C" double medusa_probe_clock_mhz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0.0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0.0;
    return khz / 1000.0;
}

extern "C" double medusa_probe_mfma_flops(int iters) {
    return (double)kNumCU * kMfmaWaves * kMfmaChains * (double)iters * 32.0 * 32.0 * 16.0 * 2.0;
}

extern "C" int medusa_probe_mfma(int iters, void *sink, void *stream) {
    if (!sink) return MEDUSA_ERR_NULL;
    if (iters < 1) return MEDUSA_ERR_PARAM;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(kNumCU), dim3(kMfmaWaves * kWave), 0,
                       (hipStream_t)stream, iters, (float *)sink);
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
}
