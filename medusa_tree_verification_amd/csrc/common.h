// Device helpers shared by the gfx950 kernels of the Medusa verify step.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "medusa_verify.h"

namespace medusa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage element types: bf16 is kept as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

constexpr int kWave = 64;
constexpr int kNumCU = 256;   // MI355X compute units (8 XCDs x 32)
constexpr int kNumXCD = 8;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two fp32 -> packed bf16 pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
// 2^x on the transcendental unit; inputs here are <= 8 or -inf
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int kPer16B = 4;
    __device__ static float to_f32(float x) { return x; }
    __device__ static float from_f32(float x) { return x; }
};
template <>
struct Elem<bf16_t> {
    static constexpr int kPer16B = 8;
    __device__ static float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
    __device__ static bf16_t from_f32(float x) { return bf16_t{f32_to_bf16(x)}; }
};

// element e (0..kPer16B-1) of a 16-byte chunk, as fp32
template <typename T>
__device__ __forceinline__ float chunk_elem(const u32x4 &c, int e);
template <>
__device__ __forceinline__ float chunk_elem<float>(const u32x4 &c, int e) { return __uint_as_float(c[e]); }
template <>
__device__ __forceinline__ float chunk_elem<bf16_t>(const u32x4 &c, int e) {
    uint32_t w = c[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// Pointer types of the direct global-to-LDS loads (global_load_lds_dwordx4:
// lane i's 16 bytes land at the wave-uniform LDS address + 16 i).
typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) const void *gbl_ptr_t;

// Streaming (non-temporal) load, for data read once: whole 128 B lines per
// instruction stream faster this way; half lines per instruction do not.
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Buffer resource over [base, base + nbytes): raw buffer loads at byte
// offsets >= nbytes return zero (hardware range check), so tails need no
// selects and addresses stay 32-bit offsets from an SGPR base.  base and
// nbytes must be wave-uniform: they are read from the first active lane (the
// compiler cannot always prove uniformity and would otherwise loop over the
// distinct values of the wave around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint64_t ua = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)ua, (short)0,
                                             __builtin_amdgcn_readfirstlane((int)nbytes),
                                             0x00020000 /* 32-bit data format, raw access */);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void st16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

// ---------------------------------------------------------------------------
// Matrix-core steps.  A "k-step" consumes one 16-byte chunk per lane of each
// operand.  Operand A supplies the output row of lane (l % N), operand B the
// output column of lane (l % N); the lanes l / N (N = 16 or 32) hold
// successive chunks along k.  Within a step, A and B lanes pair their
// elements position by position, so any consistent assignment of k indices
// to (lane group, element) gives the same dot products.
// ---------------------------------------------------------------------------

// 16x16 output tile, D[4*(l/16) + i][l%16] in acc[i].
__device__ __forceinline__ void mma16_step(f32x4 &acc, const u32x4 &a, const u32x4 &b, bf16_t) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16_step(f32x4 &acc, const u32x4 &a, const u32x4 &b, float) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc,
                                                   0, 0, 0);
}

// 32x32 output tile, D[8*(r/4) + 4*(l/32) + r%4][l%32] in acc[r].
__device__ __forceinline__ void mma32_step(f32x16 &acc, const u32x4 &a, const u32x4 &b, bf16_t) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32_step(f32x16 &acc, const u32x4 &a, const u32x4 &b, float) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc,
                                                   0, 0, 0);
}
__device__ __forceinline__ void mma32_f32_single(f32x16 &acc, float a, float b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Map the hardware block id to a logical id so that logical ids
// [x*n/8, (x+1)*n/8) all run on XCD x: neighbours in logical order then
// share an L2.  Bijective for any n.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t hw, uint32_t n) {
    const uint32_t q = n / kNumXCD, r = n % kNumXCD;
    const uint32_t x = hw % kNumXCD, k = hw / kNumXCD;
    return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// ---------------------------------------------------------------------------
// Ordered candidates: larger value first, equal values -> smaller id.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool cand_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Host-side helpers -----------------------------------------------------------
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace medusa
