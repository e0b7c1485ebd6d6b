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
// operand.  A workgroup owns 64 rows of W and a slice of K; its four waves
// split that slice and are summed in LDS in a fixed order; S workgroups
// per 64-row block split K further and leave fp32 partials that an
// epilogue kernel sums in a fixed order, so results do not depend on
// timing.  The q/k/v epilogue also applies the rotary embedding and writes
// the [B][H][T][dh] layout the tree attention reads; the output projection
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

constexpr int kGemmWaves = 4;       // waves per workgroup, each a slice of the WG's K range
constexpr int kGemmTiles = 4;       // 16-row W tiles per workgroup
constexpr int kGemmRows = 16 * kGemmTiles;
constexpr int kGemmCols = 64;       // X rows per workgroup (MT <= 4 tiles of 16)
constexpr int kGemmUnroll = 4;      // k-steps per batch of loads
constexpr int kGemmTargetWaves = 8 * kNumCU;
constexpr int kEpiThreads = 256;
constexpr int kNormThreads = 256;

struct GemmArgs {
    const void *X;        // [M][K], or [B][H][T][dh] with K = H * dh when xT > 0
    const void *W0, *W1, *W2;   // row segments of W, concatenated
    int end0, end1;       // first row of segments 1 and 2 (multiples of kGemmRows)
    float *Y;             // direct: [M][N]; otherwise partials [S][M][N]
    int M, N, K, S, MG;
    int xT, xsh;          // heads layout of X: T and log2(dh)
    int direct, accumulate;
};

// One workgroup: W rows [n0, n0 + 64) x X rows [m0, m0 + 16 MT) over the
// k-steps of split s.  Wave w takes the w-th quarter of those k-steps.
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

    const int KS = K / KSTEP, parts = a.S * kGemmWaves, part = s * kGemmWaves + wave;
    const int kb = (int)((long long)KS * part / parts), ke = (int)((long long)KS * (part + 1) / parts);

    const T *arow[kGemmTiles];
#pragma unroll
    for (int r = 0; r < kGemmTiles; ++r) {
        int n = n0 + 16 * r + c;
        n = n < N ? n : N - 1;
        arow[r] = W + (size_t)(n - segbeg) * K + g * KC;
    }
    const int xT = a.xT, xsh = a.xsh, xmask = (1 << xsh) - 1;
    const T *brow[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        int m = m0 + 16 * j + c;
        m = m < M ? m : M - 1;
        if (xT > 0) {
            const int b = m / xT, t = m - b * xT;
            brow[j] = (const T *)a.X + ((size_t)b * (K >> xsh) * xT + t) * ((size_t)1 << xsh) + g * KC;
        } else {
            brow[j] = (const T *)a.X + (size_t)m * K + g * KC;
        }
    }

    f32x4 acc[kGemmTiles][MT];
#pragma unroll
    for (int r = 0; r < kGemmTiles; ++r)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k = kb; k < ke; k += U) {
        // a short last batch loads its final step again (cached) and skips
        // the extra products, so every batch issues all its loads up front
        const int nu = ke - k < U ? ke - k : U;
        u32x4 av[kGemmTiles][U], bv[MT][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = (k + (u < nu ? u : nu - 1)) * KSTEP;
            const size_t xo = xT > 0 ? ((size_t)(kk >> xsh) * xT << xsh) + (kk & xmask) : (size_t)kk;
#pragma unroll
            for (int j = 0; j < MT; ++j) bv[j][u] = ld16(brow[j] + xo);
#pragma unroll
            for (int r = 0; r < kGemmTiles; ++r) av[r][u] = ld16(arow[r] + kk);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u < nu) {
#pragma unroll
                for (int r = 0; r < kGemmTiles; ++r)
#pragma unroll
                    for (int j = 0; j < MT; ++j) mma16_step(acc[r][j], av[r][u], bv[j][u], T{});
            }
        }
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
    float *Y = a.direct ? a.Y : a.Y + (size_t)s * M * N;
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int r = 0; r < kGemmTiles; ++r) {
        if ((r < kGemmTiles / 2) != (wave == 0)) continue;
        const int n = n0 + 16 * r + 4 * g;   // lane holds Y[m0 + 16j + c][n .. n + 3]
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const int m = m0 + 16 * j + c;
            if (m >= M || n >= N) continue;
            const f32x4 v = acc[r][j] + red[1 - wave][r * MT + j][lane];
            float *dst = Y + (size_t)m * N + n;
            if (vec) {
                f32x4 o = v;
                if (a.accumulate) o += *reinterpret_cast<const f32x4 *>(dst);
                *reinterpret_cast<f32x4 *>(dst) = o;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n + i < N) dst[i] = (a.accumulate ? dst[i] : 0.f) + v[i];
            }
        }
    }
}

// Y[i] (+)= sum over s of part[s][i], s in order
__global__ __launch_bounds__(kEpiThreads) void epi_sum_kernel(const float *__restrict__ part,
                                                              float *__restrict__ Y, size_t n,
                                                              int S, int accumulate) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x) {
        float v = part[i];
        for (int s = 1; s < S; ++s) v += part[(size_t)s * n + i];
        Y[i] = accumulate ? Y[i] + v : v;
    }
}

struct QkvEpi {
    const float *part;          // [S][M][N], N = (Hq + 2 Hkv) dh: q | k | v columns
    void *dst[3];               // q [B][Hq][T][dh], k and v [B][Hkv][T][dh]
    const int32_t *prefix_len;
    int S, M, N, T, dh, Hq, Hkv, Lcap;
    double theta;
    uint8_t depth[MEDUSA_MAX_TREE];
};

// Sum the partials of column pair (j, j + dh/2) of one head, rotate q and k
// by the angle pos * theta^(-2j/dh) (fp64) at pos = clamp(L_b) + depth(t),
// round to the dtype and store at [b][h][t][j] and [b][h][t][j + dh/2].
template <typename T>
__global__ __launch_bounds__(kEpiThreads) void qkv_epi_kernel(QkvEpi p) {
    const int half = p.dh / 2;
    const size_t pairs_row = (size_t)p.N / 2, total = (size_t)p.M * pairs_row;
    const size_t mn = (size_t)p.M * p.N;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const int m = (int)(i / pairs_row);
        const int q = (int)(i - (size_t)m * pairs_row);
        const int hd = q / half, j = q - hd * half;     // head over q | k | v, pair index
        const int seg = hd < p.Hq ? 0 : (hd < p.Hq + p.Hkv ? 1 : 2);
        const int h = seg == 0 ? hd : (seg == 1 ? hd - p.Hq : hd - p.Hq - p.Hkv);
        const int H = seg == 0 ? p.Hq : p.Hkv;
        const size_t c1 = (size_t)m * p.N + (size_t)hd * p.dh + j;
        float x1 = p.part[c1], x2 = p.part[c1 + half];
        for (int s = 1; s < p.S; ++s) {
            x1 += p.part[s * mn + c1];
            x2 += p.part[s * mn + c1 + half];
        }
        const int b = m / p.T, t = m - b * p.T;
        float y1 = x1, y2 = x2;
        if (seg < 2) {
            int L = p.prefix_len[b];
            L = L < 0 ? 0 : (L > p.Lcap ? p.Lcap : L);
            const double ang = (double)(L + p.depth[t]) * pow(p.theta, -2.0 * j / p.dh);
            const double cs = cos(ang), sn = sin(ang);
            y1 = (float)((double)x1 * cs - (double)x2 * sn);
            y2 = (float)((double)x1 * sn + (double)x2 * cs);
        }
        T *d = (T *)(seg == 0 ? p.dst[0] : (seg == 1 ? p.dst[1] : p.dst[2])) +
               (((size_t)b * H + h) * p.T + t) * p.dh;
        d[j] = Elem<T>::from_f32(y1);
        d[j + half] = Elem<T>::from_f32(y2);
    }
}

// x[m] = rmsnorm(h[m]) g rounded to the dtype, one workgroup per row.  With
// FROM_IN the row is read from the dtype input (the first block) and also
// stored to h as fp32, which starts the residual stream.
template <typename T, bool FROM_IN>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const T *__restrict__ in,
                                                               float *__restrict__ h,
                                                               const T *__restrict__ gain,
                                                               T *__restrict__ x, int d, float eps) {
    __shared__ float red[kNormThreads / kWave];
    const size_t row = (size_t)blockIdx.x * d;
    float ss = 0.f;
    for (int i = threadIdx.x; i < d; i += kNormThreads) {
        float v;
        if (FROM_IN) {
            v = Elem<T>::to_f32(in[row + i]);
            h[row + i] = v;
        } else {
            v = h[row + i];
        }
        ss += v * v;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kNormThreads / kWave; ++w) tot += red[w];
    const float inv = 1.0f / sqrtf(tot / (float)d + eps);
    for (int i = threadIdx.x; i < d; i += kNormThreads) {
        const float v = FROM_IN ? Elem<T>::to_f32(in[row + i]) : h[row + i];
        x[row + i] = Elem<T>::from_f32(v * inv * Elem<T>::to_f32(gain[i]));
    }
}

// ------------------------------------------------------------------ host
struct GemmPlan {
    int S, MG, RB, MT;
    size_t part_bytes;   // partials needed (0 when written directly)
};

// S splits of K per 64-row block, so that about kGemmTargetWaves waves run,
// each with at least two k-steps.  need_part forces partials (an epilogue
// reads them).
inline GemmPlan gemm_plan(int M, int N, int K, int kstep, bool need_part) {
    GemmPlan g;
    g.RB = (N + kGemmRows - 1) / kGemmRows;
    g.MG = (M + kGemmCols - 1) / kGemmCols;
    g.MT = M >= kGemmCols ? 4 : (M + 15) / 16;
    const double units = (double)g.RB * g.MG * kGemmWaves;
    int S = (int)(kGemmTargetWaves / units + 0.5);
    const int smax = K / kstep / (2 * kGemmWaves);
    S = S < smax ? S : smax;
    g.S = S > 1 ? S : 1;
    g.part_bytes = (need_part || g.S > 1) ? (size_t)g.S * M * N * 4 : 0;
    return g;
}

struct FwdLayout {
    size_t h, x, q, kt, vt, att, part, attn, total;
    size_t attn_bytes;
    GemmPlan qkv, wo, lm;
};

inline FwdLayout fwd_layout(int B, int T, int d, int Hq, int Hkv, int dh, int Lcap, int V,
                            int dtype) {
    const int M = B * T, es = dtype == MEDUSA_BF16 ? 2 : 4, kstep = dtype == MEDUSA_BF16 ? 32 : 16;
    FwdLayout L;
    L.qkv = gemm_plan(M, (Hq + 2 * Hkv) * dh, d, kstep, true);
    L.wo = gemm_plan(M, d, Hq * dh, kstep, false);
    L.lm = gemm_plan(M, V, d, kstep, false);
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
    L.attn_bytes = tree_attention_workspace_bytes(B, Hq, Hkv, Lcap, dh, T, dtype);
    L.attn = take(L.attn_bytes);
    L.total = off;
    return L;
}

inline unsigned grid_for(size_t n, int threads) {
    const size_t g = (n + threads - 1) / threads;
    return (unsigned)(g < 8192 ? (g > 0 ? g : 1) : 8192);
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
    const dim3 grid((unsigned)(g.RB * g.S * g.MG)), block(kGemmWaves * kWave);
    switch (g.MT) {
        case 1: hipLaunchKernelGGL((gemm_xwt_kernel<T, 1>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((gemm_xwt_kernel<T, 2>), grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL((gemm_xwt_kernel<T, 3>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((gemm_xwt_kernel<T, 4>), grid, block, 0, st, a); break;
    }
    if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    if (!a.direct && epi_sum) {
        const size_t n = (size_t)a.M * a.N;
        hipLaunchKernelGGL(epi_sum_kernel, dim3(grid_for(n, kEpiThreads)), dim3(kEpiThreads), 0, st,
                           (const float *)part, Y, n, g.S, accumulate);
        if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    }
    return MEDUSA_OK;
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
    qe.prefix_len = f.prefix_len;
    qe.S = L.qkv.S;
    qe.M = M;
    qe.N = (f.Hq + 2 * f.Hkv) * dh;
    qe.T = f.T;
    qe.dh = dh;
    qe.Hq = f.Hq;
    qe.Hkv = f.Hkv;
    qe.Lcap = f.Lcap;
    qe.theta = f.theta;
    for (int i = 0; i < MEDUSA_MAX_TREE; ++i) qe.depth[i] = 0;
    for (int n = 1; n < f.T; ++n) qe.depth[n] = (uint8_t)(qe.depth[f.parent[n]] + 1);
    const size_t kv_block = (size_t)M * f.Hkv * dh;   // one block's tree keys (or values)
    const int xsh = dh == 128 ? 7 : 6;

    for (int l = 0; l <= f.N; ++l) {
        const T *gain = (const T *)(l < f.N ? f.g[l] : f.g_final);
        if (l == 0)
            hipLaunchKernelGGL((rmsnorm_kernel<T, true>), dim3(M), dim3(kNormThreads), 0, st,
                               (const T *)f.h0, h, gain, x, f.d, f.eps);
        else
            hipLaunchKernelGGL((rmsnorm_kernel<T, false>), dim3(M), dim3(kNormThreads), 0, st,
                               (const T *)nullptr, h, gain, x, f.d, f.eps);
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
        hipLaunchKernelGGL(qkv_epi_kernel<T>, dim3(grid_for((size_t)M * qe.N / 2, kEpiThreads)),
                           dim3(kEpiThreads), 0, st, qe);
        if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;

        rc = tree_attention(ws + L.q, f.kc[l], f.vc[l], f.prefix_len, qe.dst[1], qe.dst[2],
                            f.parent, f.B, f.Hq, f.Hkv, f.Lcap, dh, f.T,
                            (float)(1.0 / sqrt((double)dh)), f.dtype, att, nullptr, ws + L.attn,
                            L.attn_bytes, st);
        if (rc != MEDUSA_OK) return rc;

        GemmArgs oa = gemm_args(att, f.wo[l], M, f.d, f.Hq * dh);
        oa.xT = f.T;
        oa.xsh = xsh;
        if ((rc = run_gemm<T>(L.wo, oa, h, part, 1, true, st)) != MEDUSA_OK) return rc;
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
    if (M * V >= (1LL << 31) || M * d >= (1LL << 31) || (long long)B * Hkv * Lcap * dh >= (1LL << 40))
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
