// Medusa heads on gfx950: H_i(h) = W2_i (SiLU(W1_i h) + h) and per-head top-s.
//
// Head equation and bias-free two-Linear head: paper explainer page,
// section "Medusa Head architecture" (equation H_i and its PyTorch listing);
// top-s candidates per head: same page, tree-attention section.
//
// Decoding with a batch of B <= 16 sequences streams K*(d*d + V*d) weights
// once per step, so both stages are HBM-bound weight streams.  Each weight
// tile of 16 output rows is the A operand of a 16x16 MFMA whose B operand is
// the (at most 16) batch columns, so one kernel serves every B <= 16 and the
// FLOPs cost nothing next to the bytes.
//
// Stage 1: the 16-row tiles over the K*d rows of W1, one per workgroup, or
//   four or five consecutive ones from four sequences on when such groups
//   fill the CUs evenly (the hidden-state loads are then shared by the
//   tiles); four waves split the d reduction; LDS sum; epilogue
//   z = SiLU(u) + h written to the workspace (bf16 rounding once, in bf16
//   mode).
// Stage 2: the row tiles of W2 (all heads' rows in one sequence) are split
//   evenly over one workgroup of four waves per CU; each wave streams a
//   contiguous range of them, in batches of 8 k-steps whose loads are issued
//   ahead of the MFMAs, starting at a per-wave rotated batch so that lockstep
//   waves hit different HBM channels.  With rows of 1 to 8 KiB the tiles
//   have 8 rows and each load instruction fetches whole 128 B lines (8 rows
//   x 128 B, non-temporal): the MFMA's second half of rows and columns takes
//   the second half of each line, and the B operand (z) sits in LDS, filled
//   by direct loads at the start: of the (at most two) heads a workgroup
//   spans for up to 8 sequences; of one head in two column groups of 8 for 9
//   to 16 (each workgroup then owns tiles of one head, and every weight load
//   feeds two MFMAs).  Measured, this streams W2 at about 7 TB/s where
//   16-row tiles (16 rows x 64 B per load, kept for other row lengths) reach
//   about 6.3; more rows in flight per wave, more waves per CU or
//   non-temporal half-line loads were all slower.  Each wave keeps per-lane
//   top-s lists of its columns, merges lists across lanes (shuffles) and
//   waves (LDS), and writes one partial list per (head, sequence) for its
//   workgroup.  A small
//   merge kernel (one workgroup per head) then reduces each head's partial
//   lists into topk_ids / topk_vals: cheaper than having the last workgroup
//   of a head merge them, whose device-scope fences cost more than a launch.
#include "common.h"

#include <mutex>

namespace medusa {
namespace {

constexpr int kSMax = MEDUSA_MAX_TOPS;   // top-s list capacity
constexpr int kS1Waves = 4;              // stage 1: waves per 16-row tile (split d)
constexpr int kS1Unroll = 8;             // stage 1: k-steps in flight per wave
constexpr int kS2Waves = 4;              // stage 2: waves per workgroup
constexpr int kS2Tiles = 4;              // stage 2: row tiles per wave pass
constexpr int kS2Unroll = 8;             // stage 2: k-steps per batch of loads
constexpr int kS2MaxWG = kNumCU;         // stage 2: workgroups (one per CU)
constexpr int kS2ZSteps = 64;            // stage 2, 8-row tiles: 128 B steps of z held in LDS per head

struct HeadsLayout {
    size_t z_off, part_off, total;
    int nh, ntph, nt, P;   // nh: streamed heads (K, plus the LM head when it rides along)
    int tr;                // stage 2 tile rows: 8 (z in LDS) or 16
    int cg;                // 8-row tiles: column groups of 8 sequences (1 or 2)
    int G;                 // workgroups per head (cg == 2: one head each), else 0
};

inline int esize(int dtype) { return dtype == MEDUSA_BF16 ? 2 : 4; }

inline HeadsLayout heads_layout(int B, int K, int d, int V, int dtype, int lm = 1) {
    HeadsLayout L;
    L.nh = K + (lm ? 1 : 0);
    // 8-row tiles when a row holds a full batch of loads (1 KiB) and z fits
    // in LDS (d * esize <= 128 B * kS2ZSteps): up to 8 sequences, z of the
    // (at most two) heads a workgroup spans; 9 to 16, z of one head in two
    // column groups, so the workgroups are dealt out G per head
    const size_t row_bytes = (size_t)d * esize(dtype);
    L.tr = row_bytes >= 128u * kS2Unroll && row_bytes <= 128u * kS2ZSteps ? 8 : 16;
    L.cg = L.tr == 8 && B > 8 ? 2 : 1;
    L.ntph = (V + L.tr - 1) / L.tr;
    L.nt = L.nh * L.ntph;
    if (L.cg == 2) {
        L.G = kS2MaxWG / L.nh < L.ntph ? kS2MaxWG / L.nh : L.ntph;
        if (L.G < 1) L.G = 1;
        L.P = L.G * L.nh;
    } else {
        L.G = 0;
        L.P = L.nt < kS2MaxWG ? L.nt : kS2MaxWG;
    }
    L.z_off = 0;
    L.part_off = align_up((size_t)B * K * d * esize(dtype), 256);
    L.total = L.part_off + align_up((size_t)L.nh * B * L.P * kSMax * 2 * sizeof(float), 256);
    return L;
}

// ------------------------------------------------------------------ stage 1
// A workgroup owns NT consecutive 16-row tiles of the K*d row space (the
// heads' W1 rows are contiguous, so a group may cross from one head into the
// next); each of its waves streams them over a quarter of d, so that every
// hidden-state fragment it loads feeds NT MFMAs (with 16 sequences those
// loads touch 16 rows each).  The quarters are summed in LDS in a fixed
// order and wave w finishes tiles w, w + 4, ...
template <typename T, int NT>
__global__ __launch_bounds__(kS1Waves *kWave) void heads_stage1_kernel(
    const T *__restrict__ hidden, const T *__restrict__ w1, T *__restrict__ z, int B, int K,
    int d) {
    constexpr int KC = Elem<T>::kPer16B;  // elements per lane per k-step
    constexpr int KSTEP = 4 * KC;         // k per step (4 lane groups)
    __shared__ f32x4 red[kS1Waves][NT][kWave];

    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int g = lane / 16, c = lane % 16;
    const size_t row0 = (size_t)blockIdx.x * NT * 16;   // first row of the K*d row space

    const int kspan = d / kS1Waves;
    const int kbeg = wave * kspan;
    const T *arow[NT];
#pragma unroll
    for (int r = 0; r < NT; ++r)
        arow[r] = w1 + (row0 + r * 16 + c) * (size_t)d + kbeg + g * KC;
    // lanes of columns >= B read column B-1: their outputs are never used, and
    // an unconditional load keeps the loop free of exec-mask branches
    const bool bcol = c < B;
    const T *brow = hidden + (size_t)(bcol ? c : B - 1) * d + kbeg + g * KC;

    // kspan = d/4 is a multiple of KSTEP (d % 128 == 0); the unrolled body
    // covers whole groups of kS1Unroll steps, the tail loop the rest.
    // Batches start at a per-wave rotated offset (spreads lockstep waves over
    // HBM channels); loads of a batch are issued ahead of its MFMAs.
    f32x4 acc[NT];
#pragma unroll
    for (int r = 0; r < NT; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int KB = KSTEP * kS1Unroll;
    const int nb = kspan / KB;
    int bi = nb > 0 ? (int)((blockIdx.x * kS1Waves + wave) % (unsigned)nb) : 0;
    for (int i = 0; i < nb; ++i) {
        const int kb = bi * KB;
        bi = bi + 1 == nb ? 0 : bi + 1;
        u32x4 a[NT][kS1Unroll], b[kS1Unroll];
#pragma unroll
        for (int u = 0; u < kS1Unroll; ++u) b[u] = ld16(brow + kb + u * KSTEP);
#pragma unroll
        for (int r = 0; r < NT; ++r)
#pragma unroll
            for (int u = 0; u < kS1Unroll; ++u) a[r][u] = ld16(arow[r] + kb + u * KSTEP);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kS1Unroll; ++u)
#pragma unroll
            for (int r = 0; r < NT; ++r) mma16_step(acc[r], a[r][u], b[u], T{});
    }
    for (int k0 = nb * KB; k0 < kspan; k0 += KSTEP) {
        const u32x4 b = ld16(brow + k0);
#pragma unroll
        for (int r = 0; r < NT; ++r) mma16_step(acc[r], ld16(arow[r] + k0), b, T{});
    }
#pragma unroll
    for (int r = 0; r < NT; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (!bcol) return;
    const T *hrow = hidden + (size_t)c * d;
    for (int r = wave; r < NT; r += kS1Waves) {
        f32x4 u = red[0][r][lane];
#pragma unroll
        for (int w = 1; w < kS1Waves; ++w) u += red[w][r][lane];
        // lane holds rows 4g + i of tile r, column (sequence) c
        const size_t R = row0 + r * 16 + 4 * g;   // row in the K*d space (a tile stays in one head)
        const int head = (int)(R / d), j0 = (int)(R % d);
        T *zrow = z + ((size_t)c * K + head) * d + j0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = u[i];
            const float silu = x / (1.0f + expf(-x));
            zrow[i] = Elem<T>::from_f32(silu + Elem<T>::to_f32(hrow[j0 + i]));
        }
    }
}

// ------------------------------------------------------------- top-s lists
template <int SM>
struct TopList {
    float v[SM];
    int id[SM];
    __device__ void clear() {
#pragma unroll
        for (int r = 0; r < SM; ++r) {
            v[r] = -INFINITY;
            id[r] = 0x7FFFFFFF;
        }
    }
    // insert keeping the first s entries sorted; entries past s stay
    // sentinels.  Branch-free: entry r keeps its place while it is ahead of
    // x (a prefix of the list, which is sorted); the first one that is not
    // gives its place to x and the ones after it move down, the s-th
    // dropping out.  A candidate behind all s entries changes nothing.
    __device__ void insert(float x, int i, int s) {
        bool keep[SM];
#pragma unroll
        for (int r = 0; r < SM; ++r) keep[r] = r >= s || cand_before(v[r], id[r], x, i);
#pragma unroll
        for (int r = SM - 1; r > 0; --r) {   // downwards: v[r - 1] is still the old entry
            const float nv = keep[r] ? v[r] : (keep[r - 1] ? x : v[r - 1]);
            const int ni = keep[r] ? id[r] : (keep[r - 1] ? i : id[r - 1]);
            v[r] = nv;
            id[r] = ni;
        }
        v[0] = keep[0] ? v[0] : x;
        id[0] = keep[0] ? id[0] : i;
    }
    __device__ void pop() {
#pragma unroll
        for (int r = 0; r < SM - 1; ++r) {
            v[r] = v[r + 1];
            id[r] = id[r + 1];
        }
        v[SM - 1] = -INFINITY;
        id[SM - 1] = 0x7FFFFFFF;
    }
};

// Merge the sorted lists held by the lanes {lane ^ m : m = m0, 2*m0, ..., 32}
// (m0 = 16: the four lanes sharing a 16x16 tile column; m0 = 1: the whole
// wave).  Afterwards every lane of a group holds in ov/oi the best s of the
// union of its group's lists.  Lists are consumed.  Ids within a group are
// distinct.
template <int SM>
__device__ void group_merge(TopList<SM> &L, int s, int m0, float (&ov)[kSMax], int (&oi)[kSMax]) {
#pragma unroll
    for (int r = 0; r < kSMax; ++r) {
        ov[r] = -INFINITY;
        oi[r] = 0x7FFFFFFF;
        if (r >= s || r >= SM) continue;
        float bv = L.v[0];
        int bi = L.id[0];
        for (int m = m0; m < kWave; m <<= 1) {
            const float v2 = __shfl_xor(bv, m);
            const int i2 = __shfl_xor(bi, m);
            if (cand_before(v2, i2, bv, bi)) {
                bv = v2;
                bi = i2;
            }
        }
        ov[r] = bv;
        oi[r] = bi;
        if (L.id[0] == bi && L.v[0] == bv) L.pop();
    }
}

// ------------------------------------------------------------------ stage 2
// acc[r] += W2 tile (tile_in_head + r) x z for r < NR: NR 16-row tiles of one
// head streamed over the full d.  Full batches of kS2Unroll k-steps issue all
// their loads ahead of their MFMAs; the batches start at batch `rot` and wrap
// around, so that waves working in lockstep sit at different column offsets
// (spreading concurrent requests over HBM channels); leftover k-steps
// (d % batch) follow one at a time.  wbase: the head's W2 plus this lane's
// chunk offset; brow: this lane's z column plus chunk offset.
template <typename T, int NR>
__device__ __forceinline__ void stream_tiles(f32x4 (&acc)[kS2Tiles], const T *__restrict__ wbase,
                                             const T *__restrict__ brow, int tile_in_head, int V,
                                             int d, int c, int rot) {
    constexpr int KC = Elem<T>::kPer16B;
    constexpr int KSTEP = 4 * KC;
    constexpr int KB = KSTEP * kS2Unroll;
    const T *arow[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        int row = (tile_in_head + r) * 16 + c;
        row = row < V ? row : V - 1;        // rows past V: loaded, never used
        arow[r] = wbase + (size_t)row * d;
    }
    const int nb = d / KB;
    int bi = nb > 0 ? rot % nb : 0;
    for (int i = 0; i < nb; ++i) {
        const int k0 = bi * KB;
        bi = bi + 1 == nb ? 0 : bi + 1;
        u32x4 a[NR][kS2Unroll], b[kS2Unroll];
#pragma unroll
        for (int u = 0; u < kS2Unroll; ++u) b[u] = ld16(brow + k0 + u * KSTEP);
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int u = 0; u < kS2Unroll; ++u) a[r][u] = ld16(arow[r] + k0 + u * KSTEP);
        // keep the whole batch of loads ahead of the MFMAs: more bytes in flight
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kS2Unroll; ++u)
#pragma unroll
            for (int r = 0; r < NR; ++r) mma16_step(acc[r], a[r][u], b[u], T{});
    }
    for (int k0 = nb * KB; k0 < d; k0 += KSTEP) {
        const u32x4 b = ld16(brow + k0);
#pragma unroll
        for (int r = 0; r < NR; ++r) mma16_step(acc[r], ld16(arow[r] + k0), b, T{});
    }
}

// acc += one 8-row W2 tile x z (up to 8 columns), over the full d.  Each
// load covers whole 128 B lines: lane (c, g) holds row c % 8 at chunk
// 4 * (c / 8) + g (16 B chunks) of every 128 B step, and its B operand is
// column c % 8 of z at the same chunk, read from LDS where zl[step * 64] is
// this lane's (stored in lane order: linear, conflict-free reads).  The
// MFMA's rows and columns 0..7 then take the first half of each step and rows
// and columns 8..15 the second, so C[i][j] + C[i + 8][j + 8] is the dot
// product of row i and column j.  Batches, rotation and the tail as in
// stream_tiles (at least one full batch: d * sizeof(T) >= 1 KiB); the weights
// are read once, so they are streamed (non-temporal loads).  The caller has
// issued the first batch into `a` (first_batch8), ahead of other work.
template <typename T>
__device__ __forceinline__ void load_batch8(u32x4 (&a)[kS2Unroll], const T *__restrict__ arow) {
    constexpr int KSTEP = 8 * Elem<T>::kPer16B;
#pragma unroll
    for (int u = 0; u < kS2Unroll; ++u) a[u] = ld16_nt(arow + u * KSTEP);
}
// CG column groups: acc[q] takes columns 8q..8q+7, whose B operands sit
// kS2ZSteps * kWave entries apart in LDS (each weight load feeds CG MFMAs).
template <typename T, int CG>
__device__ __forceinline__ void mma_batch8(f32x4 (&acc)[CG], const u32x4 (&a)[kS2Unroll],
                                           const u32x4 *zl) {
    u32x4 b[CG][kS2Unroll];
#pragma unroll
    for (int q = 0; q < CG; ++q)
#pragma unroll
        for (int u = 0; u < kS2Unroll; ++u) b[q][u] = zl[q * kS2ZSteps * kWave + u * kWave];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kS2Unroll; ++u)
#pragma unroll
        for (int q = 0; q < CG; ++q) mma16_step(acc[q], a[u], b[q][u], T{});
}
template <typename T, int CG>
__device__ __forceinline__ void stream_tile8(f32x4 (&acc)[CG], const T *__restrict__ arow,
                                             const u32x4 *zl, int d, int rot,
                                             u32x4 (&a)[kS2Unroll]) {
    constexpr int KC = Elem<T>::kPer16B;
    constexpr int KSTEP = 8 * KC;   // elements per 128 B step
    constexpr int KB = KSTEP * kS2Unroll;
    const int nb = d / KB;
    int bi = rot % nb;
    mma_batch8<T, CG>(acc, a, zl + bi * kS2Unroll * kWave);
    for (int i = 1; i < nb; ++i) {
        bi = bi + 1 == nb ? 0 : bi + 1;
        load_batch8<T>(a, arow + bi * KB);
        mma_batch8<T, CG>(acc, a, zl + bi * kS2Unroll * kWave);
    }
    for (int k0 = nb * KB; k0 < d; k0 += KSTEP) {
        const u32x4 w = ld16_nt(arow + k0);
#pragma unroll
        for (int q = 0; q < CG; ++q)
            mma16_step(acc[q], w, zl[q * kS2ZSteps * kWave + k0 / KSTEP * kWave], T{});
    }
}

// Workgroups of the stream: with G > 0, G per head (each owns a contiguous
// range of that head's tiles); otherwise the nt tiles are dealt out over P
// workgroups in order, and tile t belongs to workgroup tile_wg(t).
//
// Workgroups are dispatched round-robin over the XCDs, so hardware id w runs
// on XCD w mod 8 (the XCC id register agrees on every launch checked), and
// the odd-numbered XCDs stream this access pattern (8-row tiles of 8 KiB
// rows, whole lines) 6-9% slower than the even ones when all read at once:
// the 8-row pattern of medusa_probe_read_timed shows it, a linear stream does
// not.  The shares are weighted accordingly: kXcdShare + 1 tiles' worth on an
// even workgroup for every kXcdShare - 1 on an odd one, when every wave gets
// kXcdMinTiles tiles or more.  Same-box runs on large_vocab_typical found no
// effect of the weights themselves: with the shares inverted, or with the
// weighting switched off in this code, the stream took 730-733 us either way
// (the XCDs that finish early leave their share of the HBM bandwidth to the
// others).  A rewrite of these functions without the weighting ran 2.5%
// slower with an unchanged main loop, so this form stays, as the fastest
// build measured.  share_prefix(j, base) is the summed share of workgroups
// base .. base + j - 1.
constexpr int kXcdShare = 32;
constexpr int kXcdMinTiles = 32;
__device__ __forceinline__ long long share_prefix(int j, int base, bool wt) {
    if (!wt) return j;
    return (long long)kXcdShare * j + ((j & 1) ? ((base & 1) ? -1 : 1) : 0);
}
__device__ __forceinline__ bool xcd_weighted(int ntph, int nt, int P, int G) {
    return G > 0 ? ntph >= kXcdMinTiles * kS2Waves * G : nt >= kXcdMinTiles * kS2Waves * P;
}
// tiles [wg_beg, wg_end) of workgroup wg
__device__ __forceinline__ void wg_tiles(int wg, int ntph, int nt, int P, int G, long long &beg,
                                         long long &end) {
    const bool wt = xcd_weighted(ntph, nt, P, G);
    if (G > 0) {
        const int h = wg / G, j = wg % G;
        const long long D = share_prefix(G, h * G, wt);
        beg = (long long)h * ntph + ntph * share_prefix(j, h * G, wt) / D;
        end = (long long)h * ntph + ntph * share_prefix(j + 1, h * G, wt) / D;
    } else {
        const long long D = share_prefix(P, 0, wt);
        beg = nt * share_prefix(wg, 0, wt) / D;
        end = nt * share_prefix(wg + 1, 0, wt) / D;
    }
}
// G == 0: the workgroup whose range holds tile t (the last w with beg(w) <= t)
__device__ __forceinline__ int tile_wg(long long t, int ntph, int nt, int P) {
    if (!xcd_weighted(ntph, nt, P, 0)) return (int)(((t + 1) * P - 1) / nt);
    const long long D = share_prefix(P, 0, true);
    const long long X = ((t + 1) * D - 1) / nt;   // the largest share prefix allowed
    int w = (int)(X / kXcdShare);
    if ((w & 1) && X % kXcdShare == 0) --w;       // share_prefix(w) = kXcdShare w + 1 > X
    return w < P - 1 ? w : P - 1;
}
// the first workgroup owning a tile of head `head`, and how many own one
__device__ __forceinline__ int head_wg_first(int head, int ntph, int nt, int P, int G) {
    return G > 0 ? head * G : tile_wg((long long)head * ntph, ntph, nt, P);
}
__device__ __forceinline__ int head_wg_count(int head, int ntph, int nt, int P, int G) {
    return G > 0 ? G
                 : tile_wg((long long)head * ntph + ntph - 1, ntph, nt, P) -
                       tile_wg((long long)head * ntph, ntph, nt, P) + 1;
}

// Merge the partial top-s lists of head `head` (one per workgroup owning a
// tile of it) into topk_ids / topk_vals: wave `wave` of workgroup row
// blockIdx.y takes column blockIdx.y * kS2Waves + wave.
template <int SM>
__device__ __forceinline__ void merge_head_lists(const float2 *__restrict__ part,
                                                 int32_t *__restrict__ topk_ids,
                                                 float *__restrict__ topk_vals,
                                                 int32_t *__restrict__ root_token,
                                                 float *__restrict__ root_val, int head, int B,
                                                 int K, int s, int ntph, int nt, int P, int G,
                                                 int wave, int lane) {
    const int nparts = head_wg_count(head, ntph, nt, P, G);
    const int col = (int)blockIdx.y * kS2Waves + wave;   // one wave per (head, column)
    if (col < B) {
        TopList<SM> M;
        M.clear();
        const float2 *src = part + ((size_t)head * B + col) * P * kSMax;
        for (int p0 = 0; p0 < nparts; p0 += kWave) {
            // the lane's s entries are loaded before any is inserted
            const int p = p0 + lane;
            const float2 *lp = src + (size_t)(p < nparts ? p : nparts - 1) * kSMax;
            float2 e[kSMax];
#pragma unroll
            for (int r = 0; r < kSMax; ++r) e[r] = r < s ? lp[r] : make_float2(0.f, 0.f);
#pragma unroll
            for (int r = 0; r < kSMax; ++r) {
                const int id = (p < nparts && r < s) ? __float_as_int(e[r].y) : 0x7FFFFFFF;
                if (id != 0x7FFFFFFF) M.insert(e[r].x, id, s);
            }
        }
        float ov[kSMax];
        int oi[kSMax];
        group_merge(M, s, 1, ov, oi);
        if (lane == 0) {
            if (head == K) {   // the LM head: its argmax is the root token
                root_token[col] = oi[0];
                if (root_val) root_val[col] = ov[0];
            } else {
#pragma unroll
                for (int r = 0; r < kSMax; ++r) {
                    if (r >= s) continue;
                    topk_ids[((size_t)col * K + head) * s + r] = oi[r];
                    if (topk_vals) topk_vals[((size_t)col * K + head) * s + r] = ov[r];
                }
            }
        }
    }
}

// The row of 8-row tile `tile_in_head` that lane (c, g) streams, at its chunk.
template <typename T>
__device__ __forceinline__ const T *tile8_row(const T *wbase, int tile_in_head, int V, int d,
                                              int c, int g) {
    constexpr int KC = Elem<T>::kPer16B;
    const int r = tile_in_head * 8 + c % 8;
    return wbase + (size_t)(r < V ? r : V - 1) * d + (c / 8) * 4 * KC + g * KC;
}

// Issue the first batch (batch rot % nb) of 8-row tile t of the streamed
// heads (head K, when LM: the LM head) into a.
template <typename T, bool LM>
__device__ __forceinline__ void first_batch8(u32x4 (&a)[kS2Unroll], const T *__restrict__ w2,
                                             const T *__restrict__ w_lm, int t, int K, int V,
                                             int d, int ntph, int c, int g, int rot) {
    constexpr int KB = 8 * Elem<T>::kPer16B * kS2Unroll;
    const int h = t / ntph;
    const T *wb = LM && h == K ? w_lm : w2 + (size_t)h * V * d;
    load_batch8<T>(a, tile8_row<T>(wb, t - h * ntph, V, d, c, g) + rot % (d / KB) * KB);
}

// A wave's lists of one head into its stage slot (st[column][entry]):
// merged over the four lanes of each column, written by lane group 0.
template <int SM, int TR, int CG>
__device__ __forceinline__ void flush_lists(TopList<SM> (&L)[CG], float2 (*st)[kSMax], int s,
                                            int g, int c) {
#pragma unroll
    for (int q = 0; q < CG; ++q) {
        float ov[kSMax];
        int oi[kSMax];
        group_merge(L[q], s, 16, ov, oi);
        if (g == 0 && (TR == 16 || c < 8)) {
#pragma unroll
            for (int r = 0; r < kSMax; ++r)
                if (r < s) st[q * 8 + c][r] = make_float2(ov[r], __int_as_float(oi[r]));
        }
        L[q].clear();
    }
}

// LM: the LM head rides along as head K (a separate instantiation, so the
// plain and the root-token streams show up as different kernels in traces).
// TR: tile rows, 16 (stream_tiles, any B) or 8 (stream_tile8); CG (8-row
// tiles): column groups, 1 for up to 8 sequences, 2 for 9 to 16 (then G > 0:
// each workgroup within one head).
template <typename T, bool LM, int SM, int TR, int CG>
__global__ __launch_bounds__(kS2Waves *kWave) void heads_stage2_kernel(
    const T *__restrict__ w2, const T *__restrict__ z, const T *__restrict__ w_lm,
    const T *__restrict__ hidden, float *__restrict__ logits_out, float2 *__restrict__ part, int B,
    int K, int d, int V, int s, int ntph, int nt, int P, int G) {
    constexpr int KC = Elem<T>::kPer16B;
    // per-wave merged lists: [wave][head slot 0/1][column][s]
    __shared__ float2 stage[kS2Waves][2][16][kSMax];
    // 8-row tiles: the B operand, [slot][128 B step][lane]; a slot holds z of
    // one of the workgroup's (at most two) heads (CG 1) or one column group
    // of its one head (CG 2)
    __shared__ u32x4 zl[TR == 8 ? 2 : 1][TR == 8 ? kS2ZSteps : 1][kWave];

    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int g = lane / 16, c = lane % 16;
    const int wg = blockIdx.x;

    for (int i = threadIdx.x; i < kS2Waves * 2 * 16 * kSMax; i += blockDim.x)
        (&stage[0][0][0][0])[i] = make_float2(-INFINITY, __int_as_float(0x7FFFFFFF));

    long long wg_beg, wg_end;
    wg_tiles(wg, ntph, nt, P, G, wg_beg, wg_end);
    const int head_lo = (int)(wg_beg / ntph);
    const long long span = wg_end - wg_beg;
    const int wv = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform
    int tile = (int)(wg_beg + span * wv / kS2Waves);
    const int wend = (int)(wg_beg + span * (wv + 1) / kS2Waves);
    const int rot = (int)(((unsigned)wg * kS2Waves + wv) * 7u);
    // 8-row tiles: the first batch of each tile is issued ahead, that of the
    // wave's first tile before the z fill (whose loads then wait alongside
    // it), that of the next tile before a tile's epilogue
    u32x4 apre[kS2Unroll];
    if constexpr (TR == 8) {
        if (tile < wend) first_batch8<T, LM>(apre, w2, w_lm, tile, K, V, d, ntph, c, g, rot);
        // z chunks in lane order: entry [slot][t][q] is what lane q = 16g + c
        // multiplies in step t (column c % 8 of its group, chunk
        // 4 * (c / 8) + g); each entry row is one direct-to-LDS load of a
        // wave, all in flight at once
        const int nstep = d / (8 * KC);
        const int head_last = (int)((wg_end - 1) / ntph);
        const int nslot = CG == 2 ? 2 : head_last - head_lo + 1;
        for (int e = wv; e < nslot * nstep; e += kS2Waves) {
            const int slot = e / nstep, t = e % nstep, hd = CG == 2 ? head_lo : head_lo + slot;
            const int cc = (CG == 2 ? slot * 8 : 0) + c % 8;
            const int col = cc < B ? cc : B - 1;
            const T *src = LM && hd == K ? hidden + (size_t)col * d : z + ((size_t)col * K + hd) * d;
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src + t * 8 * KC + (c / 8) * 4 * KC + g * KC),
                                             (lds_ptr_t)&zl[slot][t][0], 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the LDS writes have landed
    }
    __syncthreads();

    const bool bcol = c < B;
    // per-lane lists: column c (16-row tiles), columns 8q + c (8-row tiles,
    // lanes c < 8; the other lanes' lists stay empty)
    TopList<SM> L[CG];
#pragma unroll
    for (int q = 0; q < CG; ++q) L[q].clear();
    int cur_head = tile < wend ? tile / ntph : -1;

    while (tile < wend) {
        const int head = tile / ntph;
        if (head != cur_head) {
            flush_lists<SM, TR, CG>(L, stage[wave][cur_head - head_lo], s, g, c);
            cur_head = head;
        }
        const bool lmh = LM && head == K;   // head K (when streamed): the LM head on the hidden state
        if constexpr (TR == 8) {
            const int tile_in_head = tile - head * ntph;
            const T *arow = tile8_row<T>(lmh ? w_lm : w2 + (size_t)head * V * d, tile_in_head, V, d, c, g);
            f32x4 acc[CG];
#pragma unroll
            for (int q = 0; q < CG; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            stream_tile8<T, CG>(acc, arow, &zl[CG == 1 ? head - head_lo : 0][0][lane], d, rot, apre);
            if (tile + 1 < wend) first_batch8<T, LM>(apre, w2, w_lm, tile + 1, K, V, d, ntph, c, g, rot);
            const int v0 = tile_in_head * 8 + 4 * g;
#pragma unroll
            for (int q = 0; q < CG; ++q) {
                // lane 16g + j (g < 2, j < 8) holds C[4g + i][j], lane 16g + j + 40 C[4g + i + 8][j + 8]
                f32x4 full;
#pragma unroll
                for (int i = 0; i < 4; ++i) full[i] = acc[q][i] + __shfl(acc[q][i], lane + 40);
                const int col = q * 8 + c;
                if (g < 2 && c < 8 && col < B) {
                    if (logits_out && head < K) {
                        float *dst = logits_out + ((size_t)col * K + head) * V + v0;
                        if (v0 + 3 < V && ((V & 3) == 0)) {
                            *reinterpret_cast<f32x4 *>(dst) = full;
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (v0 + i < V) dst[i] = full[i];
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (v0 + i < V) L[q].insert(full[i], v0 + i, s);
                }
            }
            tile += 1;
            continue;
        }
        const int head_end = (head + 1) * ntph;
        const int gend = tile + kS2Tiles < wend ? tile + kS2Tiles : wend;
        const int n = __builtin_amdgcn_readfirstlane((gend < head_end ? gend : head_end) - tile);
        const int tile_in_head = tile - head * ntph;

        f32x4 acc[kS2Tiles];
#pragma unroll
        for (int r = 0; r < kS2Tiles; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int bc = bcol ? c : B - 1;
        const T *brow = lmh ? hidden + (size_t)bc * d + g * KC
                            : z + ((size_t)bc * K + head) * d + g * KC;
        const T *wbase = lmh ? w_lm + g * KC : w2 + (size_t)head * V * d + g * KC;
        // n is wave-uniform: one straight-line body per tile count
        switch (n) {
            case 1: stream_tiles<T, 1>(acc, wbase, brow, tile_in_head, V, d, c, rot); break;
            case 2: stream_tiles<T, 2>(acc, wbase, brow, tile_in_head, V, d, c, rot); break;
            case 3: stream_tiles<T, 3>(acc, wbase, brow, tile_in_head, V, d, c, rot); break;
            default: stream_tiles<T, kS2Tiles>(acc, wbase, brow, tile_in_head, V, d, c, rot); break;
        }

        // epilogue: lane holds rows 16*tile + 4g + i of column c
#pragma unroll
        for (int r = 0; r < kS2Tiles; ++r) {
            if (r >= n) continue;
            const int v0 = (tile_in_head + r) * 16 + 4 * g;
            if (bcol) {
                if (logits_out && head < K) {
                    float *dst = logits_out + ((size_t)c * K + head) * V + v0;
                    if (v0 + 3 < V && ((V & 3) == 0)) {
                        *reinterpret_cast<f32x4 *>(dst) = acc[r];
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (v0 + i < V) dst[i] = acc[r][i];
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (v0 + i < V) L[0].insert(acc[r][i], v0 + i, s);
            }
        }
        tile += n;
    }
    if (cur_head >= 0) flush_lists<SM, TR, CG>(L, stage[wave][cur_head - head_lo], s, g, c);
    __syncthreads();

    // workgroup merge: one thread per (head slot, column)
    const int head_hi = (int)((wg_end - 1) / ntph);
    const int nslot = head_hi - head_lo + 1;
    if (threadIdx.x < nslot * 16) {
        const int slot = threadIdx.x / 16, col = threadIdx.x % 16;
        const int head = head_lo + slot;
        if (col < B) {
            float2 *dst = part + (((size_t)head * B + col) * P + (wg - head_wg_first(head, ntph, nt, P, G))) * kSMax;
            for (int r = 0; r < s; ++r) {
                float bv = -INFINITY;
                int bi = 0x7FFFFFFF, bw = -1, br = -1;
                for (int w = 0; w < kS2Waves; ++w)
                    for (int q = 0; q < s; ++q) {
                        const float2 e = stage[w][slot][col][q];
                        const int id = __float_as_int(e.y);
                        if (id == 0x7FFFFFFF) continue;
                        if (cand_before(e.x, id, bv, bi)) {
                            bv = e.x;
                            bi = id;
                            bw = w;
                            br = q;
                        }
                    }
                if (bw >= 0) stage[bw][slot][col][br] = make_float2(-INFINITY, __int_as_float(0x7FFFFFFF));
                dst[r] = make_float2(bv, __int_as_float(bi));
            }
        }
    }
}

// The final top-s of one head: the per-workgroup partial lists of the
// workgroups that own its tiles, merged with one wave per column.
template <int SM>
__global__ __launch_bounds__(kS2Waves *kWave) void heads_merge_kernel(
    const float2 *__restrict__ part, int32_t *__restrict__ topk_ids, float *__restrict__ topk_vals,
    int32_t *__restrict__ root_token, float *__restrict__ root_val, int B, int K, int s, int ntph,
    int nt, int P, int G) {
    merge_head_lists<SM>(part, topk_ids, topk_vals, root_token, root_val, (int)blockIdx.x, B, K, s,
                         ntph, nt, P, G, (int)(threadIdx.x / kWave), (int)(threadIdx.x % kWave));
}

// --------------------------------------------------------------- host side
int check_heads_args(const void *w, int B, int K, int d, int V, int s, int dtype) {
    if (!w) return MEDUSA_ERR_NULL;
    if (dtype != MEDUSA_F32 && dtype != MEDUSA_BF16) return MEDUSA_ERR_DTYPE;
    if (B < 1 || B > MEDUSA_MAX_BATCH || K < 1 || K > MEDUSA_MAX_HEADS || d < 128 || d > 16384 ||
        d % 128 != 0 || V < 1 || s < 1 || s > MEDUSA_MAX_TOPS || s > V)
        return MEDUSA_ERR_SHAPE;
    if ((long long)K * V * d >= (1LL << 62)) return MEDUSA_ERR_SHAPE;
    return MEDUSA_OK;
}

int check_ws(void *ws, size_t ws_bytes, size_t need) {
    if (!ws) return MEDUSA_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return MEDUSA_ERR_WORKSPACE;
    if (ws_bytes < need) return MEDUSA_ERR_WORKSPACE;
    return MEDUSA_OK;
}

int launch_stage1(const void *hidden, const void *w1, int B, int K, int d, int V, int dtype,
                  void *ws, hipStream_t st) {
    const HeadsLayout L = heads_layout(B, K, d, V, dtype);
    char *base = (char *)ws;
    // Four (or five) tiles per workgroup share the hidden-state loads, which
    // pays from four sequences on (a single sequence's loads are one row,
    // cheap) when the groups then fill the CUs evenly (K = 5 heads of 4096:
    // 256 groups of five, where groups of four would leave a partial round);
    // otherwise one tile each, for a fine-grained grid.
    const size_t tiles = (size_t)K * d / 16;
    const int nt = B < 4 ? 1 : (tiles / 4) % kNumCU == 0 ? 4 : (tiles / 5) % kNumCU == 0 && tiles % 5 == 0 ? 5 : 1;
    const dim3 grid((unsigned)(tiles / nt)), block(kS1Waves * kWave);
    if (dtype == MEDUSA_BF16) {
        auto *kern = nt == 4 ? heads_stage1_kernel<bf16_t, 4>
                   : nt == 5 ? heads_stage1_kernel<bf16_t, 5> : heads_stage1_kernel<bf16_t, 1>;
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const bf16_t *)hidden, (const bf16_t *)w1,
                           (bf16_t *)(base + L.z_off), B, K, d);
    } else {
        auto *kern = nt == 4 ? heads_stage1_kernel<float, 4>
                   : nt == 5 ? heads_stage1_kernel<float, 5> : heads_stage1_kernel<float, 1>;
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const float *)hidden, (const float *)w1,
                           (float *)(base + L.z_off), B, K, d);
    }
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
}

template <typename T, int TR, int CG>
auto stage2_kernel_tr(bool lm, bool s4) {
    return lm ? (s4 ? heads_stage2_kernel<T, true, 4, TR, CG> : heads_stage2_kernel<T, true, kSMax, TR, CG>)
              : (s4 ? heads_stage2_kernel<T, false, 4, TR, CG> : heads_stage2_kernel<T, false, kSMax, TR, CG>);
}
template <typename T>
auto stage2_kernel(bool lm, bool s4, int tr, int cg) {
    if (tr == 8) return cg == 2 ? stage2_kernel_tr<T, 8, 2>(lm, s4) : stage2_kernel_tr<T, 8, 1>(lm, s4);
    return stage2_kernel_tr<T, 16, 1>(lm, s4);
}

// The W2 stream with the fused per-workgroup top-s (partials into the
// workspace).  w_lm == NULL: the K Medusa heads only; otherwise the LM head
// (input: the hidden state) is streamed as head K.
int launch_stage2_stream(const void *w2, const void *w_lm, const void *hidden, int B, int K,
                         int d, int V, int s, int dtype, float *logits_out, void *ws,
                         hipStream_t st) {
    const HeadsLayout L = heads_layout(B, K, d, V, dtype, w_lm != nullptr);
    char *base = (char *)ws;
    float2 *part = (float2 *)(base + L.part_off);
    const dim3 grid((unsigned)L.P), block(kS2Waves * kWave);
    const bool lm = w_lm != nullptr;
    // lists of 4 when s <= 4 (every insert costs its capacity)
    const bool s4 = s <= 4;
    if (dtype == MEDUSA_BF16) {
        auto *kern = stage2_kernel<bf16_t>(lm, s4, L.tr, L.cg);
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const bf16_t *)w2,
                           (const bf16_t *)(base + L.z_off), (const bf16_t *)w_lm,
                           (const bf16_t *)hidden, logits_out, part, B, K, d, V, s, L.ntph, L.nt,
                           L.P, L.G);
    } else {
        auto *kern = stage2_kernel<float>(lm, s4, L.tr, L.cg);
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const float *)w2,
                           (const float *)(base + L.z_off), (const float *)w_lm,
                           (const float *)hidden, logits_out, part, B, K, d, V, s, L.ntph, L.nt,
                           L.P, L.G);
    }
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
}

// The merge of the partial lists into topk_ids / topk_vals (and, with the LM
// head, root_token / root_val).
int launch_stage2_merge(bool lm, int B, int K, int d, int V, int s, int dtype, int32_t *topk_ids,
                        float *topk_vals, int32_t *root_token, float *root_val, void *ws,
                        hipStream_t st) {
    const HeadsLayout L = heads_layout(B, K, d, V, dtype, lm);
    const float2 *part = (const float2 *)((char *)ws + L.part_off);
    hipLaunchKernelGGL(s <= 4 ? heads_merge_kernel<4> : heads_merge_kernel<kSMax>,
                       dim3((unsigned)L.nh, (unsigned)((B + kS2Waves - 1) / kS2Waves)),
                       dim3(kS2Waves * kWave), 0, st, part, topk_ids, topk_vals, root_token,
                       root_val, B, K, s, L.ntph, L.nt, L.P, L.G);
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
}

int launch_stage2(const void *w2, const void *w_lm, const void *hidden, int B, int K, int d,
                  int V, int s, int dtype, float *logits_out, int32_t *topk_ids,
                  float *topk_vals, int32_t *root_token, float *root_val, void *ws,
                  hipStream_t st) {
    const int rc = launch_stage2_stream(w2, w_lm, hidden, B, K, d, V, s, dtype, logits_out, ws, st);
    if (rc != MEDUSA_OK) return rc;
    return launch_stage2_merge(w_lm != nullptr, B, K, d, V, s, dtype, topk_ids, topk_vals,
                               root_token, root_val, ws, st);
}

}  // namespace
}  // namespace medusa

using namespace medusa;

extern "C" size_t medusa_heads_topk_workspace_bytes(int B, int K, int d, int V, int s, int dtype) {
    if (check_heads_args((const void *)1, B, K, d, V, s, dtype) != MEDUSA_OK) return 0;
    return heads_layout(B, K, d, V, dtype).total;
}

extern "C" int medusa_heads_stage1(const void *hidden, const void *w1, int B, int K, int d, int V,
                                   int s, int dtype, void *ws, size_t ws_bytes, void *stream) {
    int st = check_heads_args(w1, B, K, d, V, s, dtype);
    if (st != MEDUSA_OK) return st;
    if (!hidden) return MEDUSA_ERR_NULL;
    st = check_ws(ws, ws_bytes, heads_layout(B, K, d, V, dtype).total);
    if (st != MEDUSA_OK) return st;
    return launch_stage1(hidden, w1, B, K, d, V, dtype, ws, (hipStream_t)stream);
}

extern "C" int medusa_heads_stage2(const void *w2, int B, int K, int d, int V, int s, int dtype,
                                   float *logits_out, int32_t *topk_ids, float *topk_vals,
                                   void *ws, size_t ws_bytes, void *stream) {
    int st = check_heads_args(w2, B, K, d, V, s, dtype);
    if (st != MEDUSA_OK) return st;
    if (!topk_ids) return MEDUSA_ERR_NULL;
    st = check_ws(ws, ws_bytes, heads_layout(B, K, d, V, dtype).total);
    if (st != MEDUSA_OK) return st;
    return launch_stage2(w2, nullptr, nullptr, B, K, d, V, s, dtype, logits_out, topk_ids,
                         topk_vals, nullptr, nullptr, ws, (hipStream_t)stream);
}

extern "C" int medusa_heads_stage2_stream(const void *w2, int B, int K, int d, int V, int s,
                                          int dtype, float *logits_out, void *ws, size_t ws_bytes,
                                          void *stream) {
    int st = check_heads_args(w2, B, K, d, V, s, dtype);
    if (st != MEDUSA_OK) return st;
    st = check_ws(ws, ws_bytes, heads_layout(B, K, d, V, dtype).total);
    if (st != MEDUSA_OK) return st;
    return launch_stage2_stream(w2, nullptr, nullptr, B, K, d, V, s, dtype, logits_out, ws,
                                (hipStream_t)stream);
}

extern "C" int medusa_heads_stage2_merge(int B, int K, int d, int V, int s, int dtype,
                                         int32_t *topk_ids, float *topk_vals, void *ws,
                                         size_t ws_bytes, void *stream) {
    int st = check_heads_args((const void *)1, B, K, d, V, s, dtype);
    if (st != MEDUSA_OK) return st;
    if (!topk_ids) return MEDUSA_ERR_NULL;
    st = check_ws(ws, ws_bytes, heads_layout(B, K, d, V, dtype).total);
    if (st != MEDUSA_OK) return st;
    return launch_stage2_merge(false, B, K, d, V, s, dtype, topk_ids, topk_vals, nullptr, nullptr,
                               ws, (hipStream_t)stream);
}

extern "C" int medusa_heads_topk(const void *hidden, const void *w1, const void *w2, int B, int K,
                                 int d, int V, int s, int dtype, float *logits_out,
                                 int32_t *topk_ids, float *topk_vals, void *ws, size_t ws_bytes,
                                 void *stream) {
    int st = check_heads_args(w2, B, K, d, V, s, dtype);
    if (st != MEDUSA_OK) return st;
    if (!hidden || !w1 || !topk_ids) return MEDUSA_ERR_NULL;
    st = check_ws(ws, ws_bytes, heads_layout(B, K, d, V, dtype).total);
    if (st != MEDUSA_OK) return st;
    st = launch_stage1(hidden, w1, B, K, d, V, dtype, ws, (hipStream_t)stream);
    if (st != MEDUSA_OK) return st;
    return launch_stage2(w2, nullptr, nullptr, B, K, d, V, s, dtype, logits_out, topk_ids,
                         topk_vals, nullptr, nullptr, ws, (hipStream_t)stream);
}

extern "C" int medusa_heads_topk_root(const void *hidden, const void *w1, const void *w2,
                                      const void *w_lm, int B, int K, int d, int V, int s,
                                      int dtype, float *logits_out, int32_t *topk_ids,
                                      float *topk_vals, int32_t *root_token, float *root_val,
                                      void *ws, size_t ws_bytes, void *stream) {
    int st = check_heads_args(w2, B, K, d, V, s, dtype);
    if (st != MEDUSA_OK) return st;
    if (!hidden || !w1 || !w_lm || !topk_ids || !root_token) return MEDUSA_ERR_NULL;
    st = check_ws(ws, ws_bytes, heads_layout(B, K, d, V, dtype).total);
    if (st != MEDUSA_OK) return st;
    st = launch_stage1(hidden, w1, B, K, d, V, dtype, ws, (hipStream_t)stream);
    if (st != MEDUSA_OK) return st;
    return launch_stage2(w2, w_lm, hidden, B, K, d, V, s, dtype, logits_out, topk_ids, topk_vals,
                         root_token, root_val, ws, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// medusa_heads_topk_noalloc: medusa_heads_topk with its scratch (z and the
// per-workgroup top-s lists) in a file-scope device array instead of a
// caller workspace, for callers that cannot allocate.  Each GPU the library
// runs on holds its own copy of the array until the process ends; its
// device address is looked up once per device (with that device current)
// and kept, since the array's name in host code is not a device address.
// ---------------------------------------------------------------------------
namespace medusa {
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// This device's address of scratch, or nullptr when it cannot be found.
void *scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace medusa

extern "C" size_t medusa_heads_topk_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

extern "C" int medusa_heads_topk_noalloc(const void *hidden, const void *w1, const void *w2, int B,
                                         int K, int d, int V, int s, int dtype, float *logits_out,
                                         int32_t *topk_ids, float *topk_vals, void *stream) {
    int st = check_heads_args(w2, B, K, d, V, s, dtype);
    if (st != MEDUSA_OK) return st;
    if (!hidden || !w1 || !topk_ids) return MEDUSA_ERR_NULL;
    if (heads_layout(B, K, d, V, dtype).total > kNoAllocScratchBytes) return MEDUSA_ERR_SCRATCH;
    void *ws = scratch_for_current_device();
    if (!ws) return MEDUSA_ERR_LAUNCH;
    st = launch_stage1(hidden, w1, B, K, d, V, dtype, ws, (hipStream_t)stream);
    if (st != MEDUSA_OK) return st;
    return launch_stage2(w2, nullptr, nullptr, B, K, d, V, s, dtype, logits_out, topk_ids,
                         topk_vals, nullptr, nullptr, ws, (hipStream_t)stream);
}
