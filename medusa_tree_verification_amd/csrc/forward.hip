// Multi-layer synthetic verify forward on gfx950: N attention blocks over
// the tree's tokens, then the LM head, so that the verification logits come
// from a forward pass instead of being an input.
//
// The tree pass is one forward pass over all candidates under the tree mask
// (paper explainer page, tree-attention section); page
// "Medusa：基于多Token预测的LLM推理加速", section 5.3, runs the model once over
// the flattened tree and reads the logits of every position.  Each block
// here: x = rmsnorm(h) g (rounded to the dtype); q, k, v = x W^T; the
// rotary embedding of q and k at position L_b + depth(n) (a node sits right
// after its ancestors); tree attention over the block's cached prefix and
// the node's ancestors-or-self; h += o Wo^T with h kept in fp32.  Finally
// logits = (rmsnorm(h) g_final) W_lm^T in fp32.
//
// The projections are skinny GEMMs Y[M][N] = X[M][K] W[N][K]^T with
// M = B*T tree rows: W is streamed from HBM once (per 64 rows of X) as the
// A operand of 16x16 MFMA tiles and X, small and L2-resident, is the B
// operand.  With M > 16, X is staged through LDS once per workgroup of 128
// W rows and shared by its four waves, so that X costs few load
// instructions per W byte (the load path, not HBM, limits otherwise).  With
// more than 256 rows (bf16) the products dominate: 256 x 256 output tiles
// with both operands brought into LDS by direct loads of whole cache lines
// (the large kernel).  S workgroups per tile may split K; they leave fp32 partials that an
// epilogue kernel sums in a fixed order, so results do not depend on
// timing.  The q/k/v epilogue also applies the rotary embedding (from a
// per-call fp64 table of cos/sin at every node's position) and writes the
// [B][H][T][dh] layout the tree attention reads; the output projection
// reads the attention output in that layout directly.
#include <math.h>

#include "common.h"

extern "C" int tree_attention(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *prefix_len, const void *k_tree, const void *v_tree,
                              const int32_t *parent, int B, int Hq, int Hkv, int Lcap, int dh,
                              int T, float scale, int dtype, void *out, uint64_t *mask_out,
                              void *ws, size_t ws_bytes, void *stream);
extern "C" size_t tree_attention_workspace_bytes(int B, int Hq, int Hkv, int Lcap, int dh, int T,
                                                 int dtype);

namespace medusa {
namespace {

// Streaming kernel (any K, small M): waves split K.
constexpr int kGemmWaves = 4;       // waves per workgroup, each a slice of the WG's K range
constexpr int kGemmTiles = 4;       // 16-row W tiles per workgroup
constexpr int kGemmRows = 16 * kGemmTiles;
constexpr int kGemmCols = 64;       // X rows per workgroup of the streaming kernel (MT <= 4 tiles of 16)
constexpr int kGemmUnroll = 4;      // k-steps per batch of loads
// Staged kernel (K a multiple of one stage, 32 < M): X through LDS.
constexpr int kLdsWaves = 4;
constexpr int kLdsTW = 2;           // 16-row W tiles per wave
constexpr int kLdsRows = kLdsWaves * kLdsTW * 16;
constexpr int kLdsU = 4;            // k-steps per stage
constexpr int kMaxSplit = 8;        // K splits (partials) per row block
constexpr int kEpiThreads = 256;
constexpr int kNormThreads = 256;

struct GemmArgs {
    const void *X;        // [M][K], or [B][H][T][dh] with K = H * dh when xT > 0
    const void *W0, *W1, *W2;   // row segments of W, concatenated
    int end0, end1;       // first row of segments 1 and 2 (multiples of 64)
    float *Y;             // direct: [M][N]; otherwise partials [S][M][N]
    int M, N, K, S, MG;
    int xT, xsh;          // heads layout of X: T and log2(dh)
    int direct, accumulate;
};

// Offset of element k of an X row: plain rows, or the [B][H][T][dh] layout
// (row base at head 0; head k >> xsh sits xT rows of dh further on).
__device__ __forceinline__ int x_off(int k, int xT, int xsh) {
    return xT > 0 ? (((k >> xsh) * xT) << xsh) + (k & ((1 << xsh) - 1)) : k;
}

template <typename T>
__device__ __forceinline__ const T *x_row(const GemmArgs &a, int m) {
    if (a.xT > 0) {
        const int b = m / a.xT, t = m - b * a.xT;
        return (const T *)a.X + ((size_t)b * (a.K >> a.xsh) * a.xT + t) * ((size_t)1 << a.xsh);
    }
    return (const T *)a.X + (size_t)m * a.K;
}

// Writes a lane's 4 outputs Y[m][n .. n + 3] (direct, optionally added to
// Y) or the partial of split s.
__device__ __forceinline__ void gemm_store(const GemmArgs &a, int s, int m, int n, f32x4 v) {
    if (m >= a.M || n >= a.N) return;
    float *dst = (a.direct ? a.Y : a.Y + (size_t)s * a.M * a.N) + (size_t)m * a.N + n;
    if ((a.N & 3) == 0) {
        if (a.accumulate) v += *reinterpret_cast<const f32x4 *>(dst);
        *reinterpret_cast<f32x4 *>(dst) = v;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (n + i < a.N) dst[i] = (a.accumulate ? dst[i] : 0.f) + v[i];
    }
}

// Streaming kernel.  One workgroup: W rows [n0, n0 + 64) x X rows
// [m0, m0 + 16 MT) over the k-steps of split s; wave w takes the w-th
// quarter of them in whole batches of kGemmUnroll (the last part also the
// remainder).  Every batch issues all its loads before its MFMAs; the four
// waves' sums are added in LDS as (w0 + w2) + (w1 + w3).
template <typename T, int MT>
__global__ __launch_bounds__(kGemmWaves *kWave) void gemm_xwt_kernel(GemmArgs a) {
    constexpr int KC = Elem<T>::kPer16B;
    constexpr int KSTEP = 4 * KC;
    constexpr int U = kGemmUnroll;
    __shared__ f32x4 red[2][kGemmTiles * MT][kWave];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane / 16, c = lane % 16;
    // logical ids on one XCD are contiguous; the MG column groups of a row
    // block are neighbours, so they share that block of W through one L2
    const int lid = (int)xcd_logical_id(blockIdx.x, gridDim.x);
    const int mg = lid % a.MG;
    const int s = (lid / a.MG) % a.S;
    const int n0 = (lid / (a.MG * a.S)) * kGemmRows;
    const int m0 = mg * kGemmCols;
    const int M = a.M, N = a.N, K = a.K;
    const T *W = (const T *)(n0 >= a.end1 ? a.W2 : (n0 >= a.end0 ? a.W1 : a.W0));
    const int segbeg = n0 >= a.end1 ? a.end1 : (n0 >= a.end0 ? a.end0 : 0);

    const int KS = K / KSTEP, NB = KS / U, parts = a.S * kGemmWaves, part = s * kGemmWaves + wave;
    const int kb = (int)((long long)NB * part / parts) * U;
    const int kbe = (int)((long long)NB * (part + 1) / parts) * U;
    const int ke = part == parts - 1 ? KS : kbe;

    const T *arow[kGemmTiles];
#pragma unroll
    for (int r = 0; r < kGemmTiles; ++r) {
        int n = n0 + 16 * r + c;
        n = n < N ? n : N - 1;
        arow[r] = W + (size_t)(n - segbeg) * K + g * KC;
    }
    const int xT = a.xT, xsh = a.xsh;
    const T *brow[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        int m = m0 + 16 * j + c;
        brow[j] = x_row<T>(a, m < M ? m : M - 1) + g * KC;
    }

    f32x4 acc[kGemmTiles][MT];
#pragma unroll
    for (int r = 0; r < kGemmTiles; ++r)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    int k = kb;
    for (; k < kbe; k += U) {
        u32x4 av[kGemmTiles][U], bv[MT][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = (k + u) * KSTEP;
            const int xo = x_off(kk, xT, xsh);
#pragma unroll
            for (int j = 0; j < MT; ++j) bv[j][u] = ld16(brow[j] + xo);
#pragma unroll
            for (int r = 0; r < kGemmTiles; ++r) av[r][u] = ld16(arow[r] + kk);
        }
        // keep the whole batch of loads ahead of the MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < kGemmTiles; ++r)
#pragma unroll
                for (int j = 0; j < MT; ++j) mma16_step(acc[r][j], av[r][u], bv[j][u], T{});
    }
    for (; k < ke; ++k) {
        const int kk = k * KSTEP;
        const int xo = x_off(kk, xT, xsh);
        u32x4 av[kGemmTiles], bv[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) bv[j] = ld16(brow[j] + xo);
#pragma unroll
        for (int r = 0; r < kGemmTiles; ++r) av[r] = ld16(arow[r] + kk);
#pragma unroll
        for (int r = 0; r < kGemmTiles; ++r)
#pragma unroll
            for (int j = 0; j < MT; ++j) mma16_step(acc[r][j], av[r], bv[j], T{});
    }

    // (w0 + w2) + (w1 + w3); wave 0 finishes tiles 0-1, wave 1 tiles 2-3
    if (wave >= 2) {
#pragma unroll
        for (int r = 0; r < kGemmTiles; ++r)
#pragma unroll
            for (int j = 0; j < MT; ++j) red[wave - 2][r * MT + j][lane] = acc[r][j];
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
        for (int r = 0; r < kGemmTiles; ++r)
#pragma unroll
            for (int j = 0; j < MT; ++j) acc[r][j] += red[wave][r * MT + j][lane];
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
        for (int r = 0; r < kGemmTiles; ++r)
            if ((r < kGemmTiles / 2) != (wave == 0))
#pragma unroll
                for (int j = 0; j < MT; ++j) red[wave][r * MT + j][lane] = acc[r][j];
    }
    __syncthreads();
    if (wave >= 2) return;
#pragma unroll
    for (int r = 0; r < kGemmTiles; ++r) {
        if ((r < kGemmTiles / 2) != (wave == 0)) continue;
#pragma unroll
        for (int j = 0; j < MT; ++j)   // lane holds Y[m0 + 16j + c][n0 + 16r + 4g .. + 3]
            gemm_store(a, s, m0 + 16 * j + c, n0 + 16 * r + 4 * g,
                       acc[r][j] + red[1 - wave][r * MT + j][lane]);
    }
}

// ---- staged kernel
template <typename T, int MT>
struct LdsCfg {
    static constexpr int KC = Elem<T>::kPer16B;
    static constexpr int KSTEP = 4 * KC;
    static constexpr int U = MT >= 8 ? kLdsU / 2 : kLdsU;              // k-steps per stage
    static constexpr int SK = U * KSTEP;                               // k per stage
    static constexpr int CHUNKS = U * MT * kWave;                      // 16-B X chunks per stage
    static constexpr int XPT = CHUNKS / (kLdsWaves * kWave);           // per thread
    static_assert(CHUNKS % (kLdsWaves * kWave) == 0, "X stage split");
};

// Issue one stage's loads: this thread's X chunks first (they are waited
// for first, to be stored to LDS), then this wave's W tiles.
template <typename T, int MT, int U, int XPT>
__device__ __forceinline__ void lds_load_stage(u32x4 (&w)[kLdsTW][U], u32x4 (&xr)[XPT],
                                               const T *const (&arow)[kLdsTW],
                                               const T *const (&xrow)[XPT], const int (&koff)[XPT],
                                               int k0, int xT, int xsh) {
    constexpr int KSTEP = LdsCfg<T, MT>::KSTEP;
#pragma unroll
    for (int i = 0; i < XPT; ++i) xr[i] = ld16(xrow[i] + x_off(k0 + koff[i], xT, xsh));
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < kLdsTW; ++r) w[r][u] = ld16(arow[r] + k0 + u * KSTEP);
}

template <typename T, int MT, int U>
__device__ __forceinline__ void lds_compute_stage(f32x4 (&acc)[kLdsTW][MT],
                                                  const u32x4 (&w)[kLdsTW][U],
                                                  const u32x4 *xs, int lane) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const u32x4 xb = xs[(u * MT + j) * kWave + lane];
#pragma unroll
            for (int r = 0; r < kLdsTW; ++r) mma16_step(acc[r][j], w[r][u], xb, T{});
        }
}

// Staged kernel.  One workgroup: W rows [n0, n0 + 128) (32 per wave) x X
// rows [m0, m0 + 16 MT) over the stages of split s.  X's stage (16 MT rows
// x U k-steps: 4, or 2 with 128 rows) is loaded once per workgroup into LDS, already in the
// MFMA operand order, and read by all four waves; the next stage's X and W
// loads are issued before the current stage's MFMAs (two LDS buffers, two
// register sets for W, one barrier per stage).
template <typename T, int MT>
__global__ __launch_bounds__(kLdsWaves *kWave, 2) void gemm_lds_kernel(GemmArgs a) {
    using C = LdsCfg<T, MT>;
    __shared__ u32x4 xs[2][C::CHUNKS];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = lane / 16, c = lane % 16;
    const int lid = (int)xcd_logical_id(blockIdx.x, gridDim.x);
    const int mg = lid % a.MG, s = (lid / a.MG) % a.S, rb = lid / (a.MG * a.S);
    const int n0 = rb * kLdsRows + wave * kLdsTW * 16, m0 = mg * 16 * MT;
    const int M = a.M, N = a.N, K = a.K, xT = a.xT, xsh = a.xsh;
    // the segment of this wave's rows; a wave wholly past N (N not a
    // multiple of 32) reads row N - 1 of the last segment, never before it
    const int nsel = n0 < N ? n0 : N - 1;
    const T *W = (const T *)(nsel >= a.end1 ? a.W2 : (nsel >= a.end0 ? a.W1 : a.W0));
    const int segbeg = nsel >= a.end1 ? a.end1 : (nsel >= a.end0 ? a.end0 : 0);
    const int NST = K / C::SK;
    const int sb = NST * s / a.S, se = NST * (s + 1) / a.S;

    const T *arow[kLdsTW];
#pragma unroll
    for (int r = 0; r < kLdsTW; ++r) {
        int n = n0 + 16 * r + c;
        n = n < N ? n : N - 1;
        arow[r] = W + (size_t)(n - segbeg) * K + g * C::KC;
    }
    // X chunk q = tid + i * 256 of a stage: k-step u, column tile j, lane l
    const T *xrow[C::XPT];
    int koff[C::XPT];
#pragma unroll
    for (int i = 0; i < C::XPT; ++i) {
        const int q = tid + i * kLdsWaves * kWave;
        const int l = q % kWave, j = (q / kWave) % MT, u = q / (kWave * MT);
        const int m = m0 + 16 * j + l % 16;
        xrow[i] = x_row<T>(a, m < M ? m : M - 1);
        koff[i] = u * C::KSTEP + (l / 16) * C::KC;
    }
    f32x4 acc[kLdsTW][MT];
#pragma unroll
    for (int r = 0; r < kLdsTW; ++r)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (sb < se) {
        u32x4 wa[kLdsTW][C::U], wb[kLdsTW][C::U], xr[C::XPT];
        lds_load_stage<T, MT, C::U, C::XPT>(wa, xr, arow, xrow, koff, sb * C::SK, xT, xsh);
#pragma unroll
        for (int i = 0; i < C::XPT; ++i) xs[0][tid + i * kLdsWaves * kWave] = xr[i];
        __syncthreads();
        int st = sb, buf = 0;
        // stages alternate between the W register sets wa and wb
        while (true) {
            if (st + 1 < se) {
                lds_load_stage<T, MT, C::U, C::XPT>(wb, xr, arow, xrow, koff, (st + 1) * C::SK, xT, xsh);
                __builtin_amdgcn_sched_barrier(0);
                lds_compute_stage<T, MT, C::U>(acc, wa, xs[buf], lane);
#pragma unroll
                for (int i = 0; i < C::XPT; ++i) xs[buf ^ 1][tid + i * kLdsWaves * kWave] = xr[i];
                __syncthreads();
            } else {
                lds_compute_stage<T, MT, C::U>(acc, wa, xs[buf], lane);
                break;
            }
            ++st;
            buf ^= 1;
            if (st + 1 < se) {
                lds_load_stage<T, MT, C::U, C::XPT>(wa, xr, arow, xrow, koff, (st + 1) * C::SK, xT, xsh);
                __builtin_amdgcn_sched_barrier(0);
                lds_compute_stage<T, MT, C::U>(acc, wb, xs[buf], lane);
#pragma unroll
                for (int i = 0; i < C::XPT; ++i) xs[buf ^ 1][tid + i * kLdsWaves * kWave] = xr[i];
                __syncthreads();
            } else {
                lds_compute_stage<T, MT, C::U>(acc, wb, xs[buf], lane);
                break;
            }
            ++st;
            buf ^= 1;
        }
    }
#pragma unroll
    for (int r = 0; r < kLdsTW; ++r)
#pragma unroll
        for (int j = 0; j < MT; ++j)
            gemm_store(a, s, m0 + 16 * j + c, n0 + 16 * r + 4 * g, acc[r][j]);
}

// ---- large kernel (bf16, many rows): both operands through LDS
// One workgroup: W rows [n0, n0 + 256) x X rows [m0, m0 + 256) over the
// 64-k stages of split s.  Each stage of both operands is brought into LDS
// by direct global-to-LDS loads: one load instruction moves 8 rows x 128 B
// (8 lanes per row, whole cache lines), lane l landing at slot l of a
// kilobyte.  Row r of a 16-row tile keeps its 16-B chunk c at slot
// c ^ ((r >> 1) & 7), so that the MFMA fragment reads (row l % 16, chunk
// l / 16 of a k-step) hit 16 distinct slots per 16 lanes.  Wave w computes
// W tiles 8 (w & 1) .. + 7 against X tiles 8 (w >> 1) .. + 7 (64 products
// of 16 x 16 per k-step).  Two stage buffers: the loads of stage st + 2 go
// into stage st's buffer once every wave has read stage st (one barrier per
// stage), spread over the first quarter of the following products; the
// fragments of the next k-step are read while the current one's products
// run.  The load counter is waited on by hand (all loads of this wave are
// the stage loads), since a full barrier with fences would drain the loads
// in flight.
constexpr int kBigTile = 256;
constexpr int kBigMinRows = 256;
constexpr int kBigSK = 64;          // k per stage (two k-steps of 32)

// s_waitcnt immediates: vmcnt(0) and vmcnt(16), lgkmcnt and expcnt untouched.
// They count every vector-memory operation of the wave, so gemm_big_kernel
// may issue none but its stage loads before its last barrier
// (tests/test_kernel_resources.py checks the compiled kernel for that).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_vm16() { __builtin_amdgcn_s_waitcnt(0x4F70); }
// workgroup barrier without memory fences; the compiler may move no memory
// access across it
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kLdsWaves *kWave, 1) void gemm_big_kernel(GemmArgs a) {
    using T = bf16_t;
    __shared__ u32x4 sm[2][2][16 * 128];   // [buffer][W, X][tile * 128 + row * 8 + slot]
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lid = (int)xcd_logical_id(blockIdx.x, gridDim.x);
    const int mg = lid % a.MG, s = (lid / a.MG) % a.S, rb = lid / (a.MG * a.S);
    const int n0 = rb * kBigTile, m0 = mg * kBigTile;
    const int M = a.M, N = a.N, K = a.K, xT = a.xT, xsh = a.xsh;
    const int NST = K / kBigSK;
    const int sb = NST * s / a.S, se = NST * (s + 1) / a.S;   // se - sb >= 2

    // load instruction i of this wave: tile rows 8 (wave + 4 i) .. + 7, one
    // per 8 lanes; byte offsets from the segment (W) or X base.  The 8 rows
    // share a segment (segments start at multiples of 64); rows past N or M
    // read the last row, whose products are never stored.
    const char *wseg[8];
    uint32_t wo[8], xo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r0 = n0 + 8 * (wave + 4 * i);
        const int nsel = r0 < N ? r0 : N - 1;
        const int segbeg = nsel >= a.end1 ? a.end1 : (nsel >= a.end0 ? a.end0 : 0);
        wseg[i] = (const char *)(nsel >= a.end1 ? a.W2 : (nsel >= a.end0 ? a.W1 : a.W0));
        const int row = 8 * (wave + 4 * i) + lane / 8;
        const int chunk = (lane % 8) ^ ((row % 16) >> 1);
        int n = n0 + row;
        n = n < N ? n : N - 1;
        wo[i] = ((uint32_t)(n - segbeg) * (uint32_t)K + chunk * 8) * 2u;
        int m = m0 + row;
        m = m < M ? m : M - 1;
        xo[i] = (uint32_t)((x_row<T>(a, m) - (const T *)a.X) + chunk * 8) * 2u;
    }
    const char *Xb = (const char *)a.X;
    // byte offset of stage st in an X row: x_off without a branch (the plain
    // layout as a heads layout whose head is longer than any row)
    const int xs = xT > 0 ? xsh : 30;
    auto xstage = [&](int st) {
        const uint32_t k = (uint32_t)st * kBigSK;
        return 2u * ((((k >> xs) * (uint32_t)xT) << xs) + (k & ((1u << xs) - 1u)));
    };
    // load q (< 16) of stage st (X stage offset xk): operand q & 1, instruction q >> 1
    auto dma = [&](int st, uint32_t xk, int q) {
        const int b = st & 1, i = q >> 1;
        if (q & 1)
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Xb + (xo[i] + xk)),
                                             (lds_ptr_t)&sm[b][1][(wave + 4 * i) * kWave], 16, 0, 0);
        else
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(wseg[i] + (wo[i] + (uint32_t)st * 128u)),
                                             (lds_ptr_t)&sm[b][0][(wave + 4 * i) * kWave], 16, 0, 0);
    };
    const int wn = (wave & 1) * 8, wm = (wave >> 1) * 8;
    const int r16 = lane % 16, cg = lane / 16;
    int fo[2];   // slot of this lane's fragment in k-step u
#pragma unroll
    for (int u = 0; u < 2; ++u) fo[u] = r16 * 8 + ((4 * u + cg) ^ (r16 >> 1));
    // fragment q of k-step u of stage st: X tiles 0-7, then W tiles 0-7
    auto rd1 = [&](u32x4 (&fw)[8], u32x4 (&fx)[8], int st, int u, int q) {
        if (q < 8) fx[q] = sm[st & 1][1][(wm + q) * 128 + fo[u]];
        else fw[q - 8] = sm[st & 1][0][(wn + q - 8) * 128 + fo[u]];
    };

    f32x4 acc[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mm = [&](const u32x4 (&fw)[8], const u32x4 (&fx)[8], int r0, int r1) {
#pragma unroll
        for (int r = r0; r < r1; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) mma16_step(acc[r][j], fw[r], fx[j], T{});
    };
    u32x4 aw[8], ax[8], bw[8], bx[8];
    // Entered with stage st in registers up to the first half of k-step 1
    // (bw, bx) and stage st + 1 loaded: finishes stage st, reads and computes
    // stage st + 1 up to the same point; loads stage st + 2 when `load`.  In
    // 16 chunks of 8 products, fenced so that they issue in this order:
    // chunks 0-3 the rest of stage st, reading k-step 0 of st + 1 (and the
    // loads, 4 per chunk); 4-11 k-step 0 of st + 1, reading its k-step 1;
    // 12-15 the first half of that.
    auto body = [&](int st, bool load) {
        const uint32_t xk = xstage(st + 2);
        wait_vm0();      // stage st + 1: this wave's loads
        lds_barrier();   // ... every wave's; every wave is done with stage st
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            if (load && c < 4) {
#pragma unroll
                for (int q = 4 * c; q < 4 * c + 4; ++q) dma(st + 2, xk, q);
            }
            if (c < 4) {
#pragma unroll
                for (int q = 0; q < 4; ++q) rd1(aw, ax, st + 1, 0, 4 * c + q);
                mm(bw, bx, 4 + c, 5 + c);
            } else if (c < 12) {
#pragma unroll
                for (int q = 0; q < 2; ++q) rd1(bw, bx, st + 1, 1, 2 * (c - 4) + q);
                mm(aw, ax, c - 4, c - 3);
            } else {
                mm(bw, bx, c - 12, c - 11);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
#pragma unroll
    for (int q = 0; q < 16; ++q) dma(sb, xstage(sb), q);
#pragma unroll
    for (int q = 0; q < 16; ++q) dma(sb + 1, xstage(sb + 1), q);
    wait_vm16();     // stage sb
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 16; ++q) rd1(aw, ax, sb, 0, q);
#pragma unroll
    for (int q = 0; q < 16; ++q) rd1(bw, bx, sb, 1, q);
    mm(aw, ax, 0, 8);
    mm(bw, bx, 0, 4);
    __builtin_amdgcn_sched_barrier(0);
    int st = sb;
    for (; st + 2 < se; ++st) body(st, true);
    body(st, false);   // st = se - 2
    mm(bw, bx, 4, 8);
    wait_vm0();
    // lane holds Y[m0 + 16 (wm + j) + c][n0 + 16 (wn + r) + 4g .. + 3]
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            gemm_store(a, s, m0 + 16 * (wm + j) + r16, n0 + 16 * (wn + r) + 4 * cg, acc[r][j]);
}

// ---- epilogues
// Y[i] (+)= sum over s < NS of part[s][i], s in order; four elements per
// thread when n % 4 == 0.
template <int NS>
__global__ __launch_bounds__(kEpiThreads) void epi_sum_kernel(const float *__restrict__ part,
                                                              float *__restrict__ Y, size_t n,
                                                              int accumulate) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    if ((n & 3) == 0) {
        const size_t n4 = n / 4;
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
            f32x4 v[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) v[s] = reinterpret_cast<const f32x4 *>(part + s * n)[i];
            f32x4 t = v[0];
#pragma unroll
            for (int s = 1; s < NS; ++s) t += v[s];
            f32x4 *y = reinterpret_cast<f32x4 *>(Y) + i;
            *y = accumulate ? *y + t : t;
        }
    } else {
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
            float v[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) v[s] = part[s * n + i];
            float t = v[0];
#pragma unroll
            for (int s = 1; s < NS; ++s) t += v[s];
            Y[i] = accumulate ? Y[i] + t : t;
        }
    }
}

struct QkvEpi {
    const float *part;          // [S][M][N], N = (Hq + 2 Hkv) dh: q | k | v columns
    const double2 *tab;         // rotary table [M][dh/2]
    void *dst[3];               // q [B][Hq][T][dh], k and v [B][Hkv][T][dh]
    int M, N, T, dh, Hq, Hkv;
};

// Sum the partials of column pair (j, j + dh/2) of one head, rotate q and k
// (x1 cos - x2 sin, x1 sin + x2 cos in fp64), round to the dtype and store
// at [b][h][t][j] and [b][h][t][j + dh/2].
template <typename T, int NS>
__global__ __launch_bounds__(kEpiThreads) void qkv_epi_kernel(QkvEpi p) {
    const int half = p.dh / 2, pairs_row = p.N / 2, total = p.M * pairs_row;
    const size_t mn = (size_t)p.M * p.N;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
        const int m = i / pairs_row, q = i - m * pairs_row;
        const int hd = q / half, j = q - hd * half;     // head over q | k | v, pair index
        const int seg = hd < p.Hq ? 0 : (hd < p.Hq + p.Hkv ? 1 : 2);
        const int h = seg == 0 ? hd : (seg == 1 ? hd - p.Hq : hd - p.Hq - p.Hkv);
        const int H = seg == 0 ? p.Hq : p.Hkv;
        const size_t c1 = (size_t)m * p.N + hd * p.dh + j;
        float a1[NS], a2[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            a1[s] = p.part[s * mn + c1];
            a2[s] = p.part[s * mn + c1 + half];
        }
        float x1 = a1[0], x2 = a2[0];
#pragma unroll
        for (int s = 1; s < NS; ++s) {
            x1 += a1[s];
            x2 += a2[s];
        }
        const int b = m / p.T, t = m - b * p.T;
        float y1 = x1, y2 = x2;
        if (seg < 2) {
            const double2 cs = p.tab[m * half + j];
            y1 = (float)((double)x1 * cs.x - (double)x2 * cs.y);
            y2 = (float)((double)x1 * cs.y + (double)x2 * cs.x);
        }
        T *d = (T *)(seg == 0 ? p.dst[0] : (seg == 1 ? p.dst[1] : p.dst[2])) +
               (((size_t)b * H + h) * p.T + t) * p.dh;
        d[j] = Elem<T>::from_f32(y1);
        d[j + half] = Elem<T>::from_f32(y2);
    }
}

// ---- RMSNorm
template <typename T>
__device__ __forceinline__ f32x4 load4(const T *p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float *p) {
    return *reinterpret_cast<const f32x4 *>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16_t>(const bf16_t *p) {
    const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
}
template <typename T>
__device__ __forceinline__ void store4(T *p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float *p, f32x4 v) {
    *reinterpret_cast<f32x4 *>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *p, f32x4 v) {
    *reinterpret_cast<u32x2 *>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

constexpr int kNormU = 4;   // groups of 4 elements per thread per pass step

struct NormArgs {
    const void *in;             // FROM_IN: the first block's input rows [M][d] (dtype)
    float *h;                   // fp32 residual stream [M][d]
    const float *part;          // NS > 0: output-projection partials [NS][M][d]
    size_t md;                  // M * d
    const void *gain;           // [d] dtype
    void *x;                    // normalised rows [M][d] (dtype)
    int d;
    float eps;
    // rotary table, written when tab != nullptr: row m's dh/2 (cos, sin)
    double2 *tab;
    const int32_t *prefix_len;
    int T, dh, Lcap;
    double theta;
    uint8_t depth[MEDUSA_MAX_TREE];
};

// x[m] = rmsnorm(h[m]) g rounded to the dtype, one workgroup per row, four
// elements per thread access with kNormU accesses in flight.  The residual
// update comes first: with FROM_IN the row is read from the dtype input (the
// first block) and starts the fp32 residual stream; with NS > 0 the previous
// block's output-projection partials are summed (in split order) and added
// to h.  h is stored back in both cases; every thread reads back only what
// it wrote itself.  The first block's launch also writes row m of the
// rotary table: cos and sin of pos * theta^(-2j/dh) at
// pos = clamp(L_b, 0, Lcap) + depth(t), in fp64 (the same for every block).
template <typename T, bool FROM_IN, int NS>
__global__ __launch_bounds__(kNormThreads) void norm_kernel(NormArgs a) {
    __shared__ float red[kNormThreads / kWave];
    const int m = blockIdx.x;
    if (a.tab && (int)threadIdx.x < a.dh / 2) {
        const int j = threadIdx.x, b = m / a.T, t = m - b * a.T;
        int L = a.prefix_len[b];
        L = L < 0 ? 0 : (L > a.Lcap ? a.Lcap : L);
        const double ang = (double)(L + a.depth[t]) * pow(a.theta, -2.0 * j / a.dh);
        double sn, cs;
        sincos(ang, &sn, &cs);
        a.tab[(size_t)m * (a.dh / 2) + j] = make_double2(cs, sn);
    }
    const size_t row = (size_t)m * a.d;
    const int d4 = a.d / 4;
    float *h = a.h;
    float ss = 0.f;
    for (int b = 0; b < d4; b += kNormU * kNormThreads) {
        f32x4 v[kNormU], pv[kNormU][NS > 0 ? NS : 1];
#pragma unroll
        for (int u = 0; u < kNormU; ++u) {
            const int c4 = b + u * kNormThreads + threadIdx.x;
            const int cc = c4 < d4 ? c4 : d4 - 1;
            v[u] = FROM_IN ? load4<T>((const T *)a.in + row + 4 * cc) : load4<float>(h + row + 4 * cc);
#pragma unroll
            for (int s = 0; s < NS; ++s) pv[u][s] = load4<float>(a.part + s * a.md + row + 4 * cc);
        }
#pragma unroll
        for (int u = 0; u < kNormU; ++u) {
            const int c4 = b + u * kNormThreads + threadIdx.x;
            if (c4 >= d4) continue;
            if (NS > 0) {
                f32x4 t = pv[u][0];
#pragma unroll
                for (int s = 1; s < NS; ++s) t += pv[u][s];
                v[u] += t;
            }
            if (FROM_IN || NS > 0) store4<float>(h + row + 4 * c4, v[u]);
            ss += v[u][0] * v[u][0] + v[u][1] * v[u][1] + v[u][2] * v[u][2] + v[u][3] * v[u][3];
        }
    }
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) ss += __shfl_xor(ss, mm);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kNormThreads / kWave; ++w) tot += red[w];
    const float inv = 1.0f / sqrtf(tot / (float)a.d + a.eps);
    for (int b = 0; b < d4; b += kNormU * kNormThreads) {
        f32x4 v[kNormU], gv[kNormU];
#pragma unroll
        for (int u = 0; u < kNormU; ++u) {
            const int c4 = b + u * kNormThreads + threadIdx.x;
            const int cc = c4 < d4 ? c4 : d4 - 1;
            v[u] = load4<float>(h + row + 4 * cc);
            gv[u] = load4<T>((const T *)a.gain + 4 * cc);
        }
#pragma unroll
        for (int u = 0; u < kNormU; ++u) {
            const int c4 = b + u * kNormThreads + threadIdx.x;
            if (c4 < d4) store4<T>((T *)a.x + row + 4 * c4, v[u] * inv * gv[u]);
        }
    }
}

// ------------------------------------------------------------------ host
struct GemmPlan {
    bool big, staged;
    int S, MG, RB, MT;
    size_t part_bytes;   // partials needed (0 when written directly)
};

// The large kernel for bf16 with more than kBigMinRows rows and K a whole
// number of its stages; else the staged kernel when K is a whole number of
// stages and M > 16 (it pays when X is read by many tiles); else the
// streaming kernel.  S splits of K per tile when the tiles alone leave most
// CUs idle (the large kernel: as many as fit in one round of the CUs), each
// split keeping at least four stages (batches per wave, eight stages for
// the large kernel); at most kMaxSplit.  need_part forces partials (an
// epilogue reads them).
inline GemmPlan gemm_plan(int M, int N, int K, int kstep, bool bf16, bool need_part) {
    GemmPlan g;
    const int KS = K / kstep;
    // (32-bit byte offsets in the large kernel: N K < 2^31)
    g.big = bf16 && M > kBigMinRows && K % kBigSK == 0 && K / kBigSK >= 2 &&
            (long long)N * K < (1LL << 31);
    if (g.big) {
        g.staged = false;
        g.MT = 0;
        g.RB = (N + kBigTile - 1) / kBigTile;
        g.MG = (M + kBigTile - 1) / kBigTile;
        const int units = g.RB * g.MG, smax = K / kBigSK / 8;
        int S = units >= 3 * kNumCU / 4 ? 1 : kNumCU / units;
        S = S < smax ? S : smax;
        S = S < kMaxSplit ? S : kMaxSplit;
        g.S = S > 1 ? S : 1;
        g.part_bytes = (need_part || g.S > 1) ? (size_t)g.S * M * N * 4 : 0;
        return g;
    }
    const int mt = M >= kGemmCols ? 4 : (M + 15) / 16;
    g.staged = mt >= 2 && KS % kLdsU == 0;
    // staged with more than 64 rows: 128 X rows per workgroup (W read from
    // L2 once per 128 rows instead of per 64)
    g.MT = g.staged && M > kGemmCols ? 8 : mt;
    const int cols = g.staged ? 16 * g.MT : kGemmCols;
    g.MG = (M + cols - 1) / cols;
    int smax, S;
    if (g.staged) {
        g.RB = (N + kLdsRows - 1) / kLdsRows;
        const int units = g.RB * g.MG;
        S = units >= 3 * kNumCU / 4 ? 1 : (2 * kNumCU + units / 2) / units;
        smax = KS / (g.MT >= 8 ? kLdsU / 2 : kLdsU) / 4;
    } else {
        g.RB = (N + kGemmRows - 1) / kGemmRows;
        const int units = g.RB * g.MG;
        S = units >= 3 * kNumCU / 4 ? 1 : (2 * kNumCU + units / 2) / units;
        smax = KS / kGemmUnroll / kGemmWaves;
    }
    S = S < smax ? S : smax;
    S = S < kMaxSplit ? S : kMaxSplit;
    g.S = S > 1 ? S : 1;
    g.part_bytes = (need_part || g.S > 1) ? (size_t)g.S * M * N * 4 : 0;
    return g;
}

struct FwdLayout {
    size_t h, x, q, kt, vt, att, part, tab, attn, total;
    size_t attn_bytes;
    GemmPlan qkv, wo, lm;
};

inline FwdLayout fwd_layout(int B, int T, int d, int Hq, int Hkv, int dh, int Lcap, int V,
                            int dtype) {
    const int M = B * T, es = dtype == MEDUSA_BF16 ? 2 : 4, kstep = dtype == MEDUSA_BF16 ? 32 : 16;
    FwdLayout L;
    const bool bf16 = dtype == MEDUSA_BF16;
    L.qkv = gemm_plan(M, (Hq + 2 * Hkv) * dh, d, kstep, bf16, true);
    L.wo = gemm_plan(M, d, Hq * dh, kstep, bf16, false);
    L.lm = gemm_plan(M, V, d, kstep, bf16, false);
    size_t part = L.qkv.part_bytes;
    part = part > L.wo.part_bytes ? part : L.wo.part_bytes;
    part = part > L.lm.part_bytes ? part : L.lm.part_bytes;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    L.h = take((size_t)M * d * 4);
    L.x = take((size_t)M * d * es);
    L.q = take((size_t)M * Hq * dh * es);
    L.kt = take((size_t)M * Hkv * dh * es);
    L.vt = take((size_t)M * Hkv * dh * es);
    L.att = take((size_t)M * Hq * dh * es);
    L.part = take(part);
    L.tab = take((size_t)M * (dh / 2) * sizeof(double2));
    L.attn_bytes = tree_attention_workspace_bytes(B, Hq, Hkv, Lcap, dh, T, dtype);
    L.attn = take(L.attn_bytes);
    L.total = off;
    return L;
}

inline unsigned grid_for(size_t n, int threads) {
    const size_t g = (n + threads - 1) / threads;
    return (unsigned)(g < 8192 ? (g > 0 ? g : 1) : 8192);
}

template <typename T, int MT>
void launch_gemm_kernel(const GemmPlan &g, const GemmArgs &a, hipStream_t st) {
    if (g.big) {
        if constexpr (std::is_same<T, bf16_t>::value)
            hipLaunchKernelGGL(gemm_big_kernel, dim3((unsigned)(g.RB * g.S * g.MG)),
                               dim3(kLdsWaves * kWave), 0, st, a);
    } else if (g.staged)
        hipLaunchKernelGGL((gemm_lds_kernel<T, MT < 2 ? 2 : MT>), dim3((unsigned)(g.RB * g.S * g.MG)),
                           dim3(kLdsWaves * kWave), 0, st, a);
    else
        hipLaunchKernelGGL((gemm_xwt_kernel<T, MT < 4 ? MT : 4>), dim3((unsigned)(g.RB * g.S * g.MG)),
                           dim3(kGemmWaves * kWave), 0, st, a);
}

template <int NS>
void launch_epi_sum(const float *part, float *Y, size_t n, int accumulate, hipStream_t st) {
    const size_t work = (n & 3) == 0 ? n / 4 : n;
    hipLaunchKernelGGL(epi_sum_kernel<NS>, dim3(grid_for(work, kEpiThreads)), dim3(kEpiThreads), 0,
                       st, part, Y, n, accumulate);
}

// Y (+)= X W^T through the plan: direct when one split and no epilogue,
// else partials in `part` and (for plain sums) the sum epilogue.
template <typename T>
int run_gemm(const GemmPlan &g, GemmArgs a, float *Y, float *part, int accumulate, bool epi_sum,
             hipStream_t st) {
    a.S = g.S;
    a.MG = g.MG;
    a.direct = g.part_bytes == 0;
    a.Y = a.direct ? Y : part;
    a.accumulate = a.direct ? accumulate : 0;
    switch (g.MT) {
        case 1: launch_gemm_kernel<T, 1>(g, a, st); break;
        case 2: launch_gemm_kernel<T, 2>(g, a, st); break;
        case 3: launch_gemm_kernel<T, 3>(g, a, st); break;
        case 4: launch_gemm_kernel<T, 4>(g, a, st); break;
        default: launch_gemm_kernel<T, 8>(g, a, st); break;
    }
    if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    if (!a.direct && epi_sum) {
        const size_t n = (size_t)a.M * a.N;
        switch (g.S) {
            case 1: launch_epi_sum<1>(part, Y, n, accumulate, st); break;
            case 2: launch_epi_sum<2>(part, Y, n, accumulate, st); break;
            case 3: launch_epi_sum<3>(part, Y, n, accumulate, st); break;
            case 4: launch_epi_sum<4>(part, Y, n, accumulate, st); break;
            case 5: launch_epi_sum<5>(part, Y, n, accumulate, st); break;
            case 6: launch_epi_sum<6>(part, Y, n, accumulate, st); break;
            case 7: launch_epi_sum<7>(part, Y, n, accumulate, st); break;
            default: launch_epi_sum<8>(part, Y, n, accumulate, st); break;
        }
        if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    }
    return MEDUSA_OK;
}

template <typename T>
void launch_qkv_epi(int S, const QkvEpi &qe, hipStream_t st) {
    const dim3 grid(grid_for((size_t)qe.M * qe.N / 2, kEpiThreads)), block(kEpiThreads);
    switch (S) {
        case 1: hipLaunchKernelGGL((qkv_epi_kernel<T, 1>), grid, block, 0, st, qe); break;
        case 2: hipLaunchKernelGGL((qkv_epi_kernel<T, 2>), grid, block, 0, st, qe); break;
        case 3: hipLaunchKernelGGL((qkv_epi_kernel<T, 3>), grid, block, 0, st, qe); break;
        case 4: hipLaunchKernelGGL((qkv_epi_kernel<T, 4>), grid, block, 0, st, qe); break;
        case 5: hipLaunchKernelGGL((qkv_epi_kernel<T, 5>), grid, block, 0, st, qe); break;
        case 6: hipLaunchKernelGGL((qkv_epi_kernel<T, 6>), grid, block, 0, st, qe); break;
        case 7: hipLaunchKernelGGL((qkv_epi_kernel<T, 7>), grid, block, 0, st, qe); break;
        default: hipLaunchKernelGGL((qkv_epi_kernel<T, 8>), grid, block, 0, st, qe); break;
    }
}

inline GemmArgs gemm_args(const void *X, const void *W, int M, int N, int K) {
    GemmArgs a;
    a.X = X;
    a.W0 = a.W1 = a.W2 = W;
    a.end0 = a.end1 = N;
    a.M = M;
    a.N = N;
    a.K = K;
    a.xT = 0;
    a.xsh = 0;
    return a;
}

struct FwdArgs {
    const void *h0;
    int N;
    const void *const *g, *const *wq, *const *wk, *const *wv, *const *wo;
    const void *g_final, *w_lm;
    const void *const *kc, *const *vc;
    const int32_t *prefix_len, *parent;
    int B, T, d, Hq, Hkv, dh, Lcap, V, dtype;
    double theta;
    float eps;
    float *logits, *hidden;
    void *k_tree_out, *v_tree_out;
};

template <typename T>
int run_forward(const FwdArgs &f, char *ws, hipStream_t st) {
    const FwdLayout L = fwd_layout(f.B, f.T, f.d, f.Hq, f.Hkv, f.dh, f.Lcap, f.V, f.dtype);
    const int M = f.B * f.T, dh = f.dh;
    float *h = f.hidden ? f.hidden : (float *)(ws + L.h);
    T *x = (T *)(ws + L.x);
    T *att = (T *)(ws + L.att);
    float *part = (float *)(ws + L.part);
    int rc;

    QkvEpi qe;
    qe.part = part;
    qe.tab = (const double2 *)(ws + L.tab);
    qe.M = M;
    qe.N = (f.Hq + 2 * f.Hkv) * dh;
    qe.T = f.T;
    qe.dh = dh;
    qe.Hq = f.Hq;
    qe.Hkv = f.Hkv;
    const size_t kv_block = (size_t)M * f.Hkv * dh;   // one block's tree keys (or values)
    const int xsh = dh == 128 ? 7 : 6;

    NormArgs na;
    na.in = f.h0;
    na.h = h;
    na.part = part;
    na.md = (size_t)M * f.d;
    na.x = x;
    na.d = f.d;
    na.eps = f.eps;
    na.tab = nullptr;
    na.prefix_len = f.prefix_len;
    na.T = f.T;
    na.dh = dh;
    na.Lcap = f.Lcap;
    na.theta = f.theta;
    for (int i = 0; i < MEDUSA_MAX_TREE; ++i) na.depth[i] = 0;
    for (int n = 1; n < f.T; ++n) na.depth[n] = (uint8_t)(na.depth[f.parent[n]] + 1);
    // the output projection's partials (when it splits K) are added to h by
    // the next norm
    const int wo_ns = L.wo.part_bytes ? L.wo.S : 0;

    for (int l = 0; l <= f.N; ++l) {
        na.gain = l < f.N ? f.g[l] : f.g_final;
        na.tab = l == 0 && f.N > 0 ? (double2 *)(ws + L.tab) : nullptr;
        const dim3 ng((unsigned)M), nb(kNormThreads);
        if (l == 0) {
            hipLaunchKernelGGL((norm_kernel<T, true, 0>), ng, nb, 0, st, na);
        } else {
            switch (wo_ns) {
                case 0: hipLaunchKernelGGL((norm_kernel<T, false, 0>), ng, nb, 0, st, na); break;
                case 1: hipLaunchKernelGGL((norm_kernel<T, false, 1>), ng, nb, 0, st, na); break;
                case 2: hipLaunchKernelGGL((norm_kernel<T, false, 2>), ng, nb, 0, st, na); break;
                case 3: hipLaunchKernelGGL((norm_kernel<T, false, 3>), ng, nb, 0, st, na); break;
                case 4: hipLaunchKernelGGL((norm_kernel<T, false, 4>), ng, nb, 0, st, na); break;
                case 5: hipLaunchKernelGGL((norm_kernel<T, false, 5>), ng, nb, 0, st, na); break;
                case 6: hipLaunchKernelGGL((norm_kernel<T, false, 6>), ng, nb, 0, st, na); break;
                case 7: hipLaunchKernelGGL((norm_kernel<T, false, 7>), ng, nb, 0, st, na); break;
                default: hipLaunchKernelGGL((norm_kernel<T, false, 8>), ng, nb, 0, st, na); break;
            }
        }
        if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
        if (l == f.N) break;

        GemmArgs qa = gemm_args(x, f.wq[l], M, qe.N, f.d);
        qa.W1 = f.wk[l];
        qa.W2 = f.wv[l];
        qa.end0 = f.Hq * dh;
        qa.end1 = (f.Hq + f.Hkv) * dh;
        if ((rc = run_gemm<T>(L.qkv, qa, nullptr, part, 0, false, st)) != MEDUSA_OK) return rc;
        qe.dst[0] = ws + L.q;
        qe.dst[1] = f.k_tree_out ? (T *)f.k_tree_out + l * kv_block : (T *)(ws + L.kt);
        qe.dst[2] = f.v_tree_out ? (T *)f.v_tree_out + l * kv_block : (T *)(ws + L.vt);
        launch_qkv_epi<T>(L.qkv.S, qe, st);
        if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;

        rc = tree_attention(ws + L.q, f.kc[l], f.vc[l], f.prefix_len, qe.dst[1], qe.dst[2],
                            f.parent, f.B, f.Hq, f.Hkv, f.Lcap, dh, f.T,
                            (float)(1.0 / sqrt((double)dh)), f.dtype, att, nullptr, ws + L.attn,
                            L.attn_bytes, st);
        if (rc != MEDUSA_OK) return rc;

        GemmArgs oa = gemm_args(att, f.wo[l], M, f.d, f.Hq * dh);
        oa.xT = f.T;
        oa.xsh = xsh;
        if ((rc = run_gemm<T>(L.wo, oa, h, part, 1, false, st)) != MEDUSA_OK) return rc;
    }
    return run_gemm<T>(L.lm, gemm_args(x, f.w_lm, M, f.V, f.d), f.logits, part, 0, true, st);
}

}  // namespace
}  // namespace medusa

using namespace medusa;

static int check_fwd(int N, int B, int T, int d, int Hq, int Hkv, int dh, int Lcap, int V,
                     int dtype) {
    if (dtype != MEDUSA_F32 && dtype != MEDUSA_BF16) return MEDUSA_ERR_DTYPE;
    const int kstep = dtype == MEDUSA_BF16 ? 32 : 16;
    if (N < 0 || N > MEDUSA_MAX_LAYERS || B < 1 || T < 1 || T > MEDUSA_MAX_TREE || d < kstep ||
        d % kstep != 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || (dh != 64 && dh != 128) ||
        Lcap < 0 || V < 1)
        return MEDUSA_ERR_SHAPE;
    const long long M = (long long)B * T;
    if (M * V >= (1LL << 31) || M * d >= (1LL << 31) || M * (Hq + 2 * Hkv) * dh >= (1LL << 31) ||
        (long long)B * Hkv * Lcap * dh >= (1LL << 40))
        return MEDUSA_ERR_SHAPE;
    return MEDUSA_OK;
}

extern "C" size_t medusa_verify_forward_workspace_bytes(int B, int T, int d, int Hq, int Hkv,
                                                        int dh, int Lcap, int V, int dtype) {
    if (check_fwd(0, B, T, d, Hq, Hkv, dh, Lcap, V, dtype) != MEDUSA_OK) return 0;
    return fwd_layout(B, T, d, Hq, Hkv, dh, Lcap, V, dtype).total;
}

extern "C" int medusa_verify_forward(
    const void *h0, int N, const void *const *g, const void *const *wq, const void *const *wk,
    const void *const *wv, const void *const *wo, const void *g_final, const void *w_lm,
    const void *const *k_caches, const void *const *v_caches, const int32_t *prefix_len,
    const int32_t *parent, int B, int T, int d, int Hq, int Hkv, int dh, int Lcap, int V,
    int dtype, double theta, float eps, float *logits, float *hidden_out, void *k_tree_out,
    void *v_tree_out, void *ws, size_t ws_bytes, void *stream) {
    int st = check_fwd(N, B, T, d, Hq, Hkv, dh, Lcap, V, dtype);
    if (st != MEDUSA_OK) return st;
    if (!h0 || !g_final || !w_lm || !prefix_len || !parent || !logits) return MEDUSA_ERR_NULL;
    if (N > 0 && (!g || !wq || !wk || !wv || !wo || !k_caches || !v_caches)) return MEDUSA_ERR_NULL;
    for (int l = 0; l < N; ++l)
        if (!g[l] || !wq[l] || !wk[l] || !wv[l] || !wo[l] || !k_caches[l] || !v_caches[l])
            return MEDUSA_ERR_NULL;
    if (!(theta > 0.0) || theta == INFINITY || !(eps >= 0.f) || eps == INFINITY)
        return MEDUSA_ERR_PARAM;
    if (parent[0] != -1) return MEDUSA_ERR_TREE;
    for (int n = 1; n < T; ++n)
        if (parent[n] < 0 || parent[n] >= n) return MEDUSA_ERR_TREE;
    const FwdLayout L = fwd_layout(B, T, d, Hq, Hkv, dh, Lcap, V, dtype);
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < L.total) return MEDUSA_ERR_WORKSPACE;
    FwdArgs f;
    f.h0 = h0;
    f.N = N;
    f.g = g;
    f.wq = wq;
    f.wk = wk;
    f.wv = wv;
    f.wo = wo;
    f.g_final = g_final;
    f.w_lm = w_lm;
    f.kc = k_caches;
    f.vc = v_caches;
    f.prefix_len = prefix_len;
    f.parent = parent;
    f.B = B;
    f.T = T;
    f.d = d;
    f.Hq = Hq;
    f.Hkv = Hkv;
    f.dh = dh;
    f.Lcap = Lcap;
    f.V = V;
    f.dtype = dtype;
    f.theta = theta;
    f.eps = eps;
    f.logits = logits;
    f.hidden = hidden_out;
    f.k_tree_out = k_tree_out;
    f.v_tree_out = v_tree_out;
    hipStream_t s = (hipStream_t)stream;
    return dtype == MEDUSA_BF16 ? run_forward<bf16_t>(f, (char *)ws, s)
                                : run_forward<float>(f, (char *)ws, s);
}
