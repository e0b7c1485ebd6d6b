// Peak probes: the two ceilings the verify step's roofline is measured
// against, measured on the device itself (the published MI355X figures are
// 8 TB/s of HBM3E and 2.5 PFLOP/s of dense bf16 MFMA).
//
//  - medusa_probe_read: a linear stream of 16-byte non-temporal loads over a
//    caller buffer, every byte read once, four waves per CU with eight loads
//    (8 KiB of whole 128 B lines per wave) in flight: the fastest read shape
//    measured (plain loads, or sixteen waves per CU, stream about 15% slower);
//    the loaded words are folded into one value per thread so that no load
//    can be dropped.
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

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4 *__restrict__ src,
                                                                   size_t n16, uint32_t *sink) {
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

extern "C" int medusa_probe_read(const void *buf, size_t bytes, void *sink, void *stream) {
    if (!buf || !sink) return MEDUSA_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0) return MEDUSA_ERR_SHAPE;
    hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeWG), dim3(kProbeThreads), 0,
                       (hipStream_t)stream, (const u32x4 *)buf, bytes / 16, (uint32_t *)sink);
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
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
