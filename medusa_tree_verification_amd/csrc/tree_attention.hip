// Tree attention on gfx950: every candidate-tree node attends to the whole
// KV-cache prefix of its sequence plus its own tree ancestors and itself, in
// one pass (paper explainer page, tree-attention section: the ancestor mask
// lets all candidate paths be verified in a single forward pass without
// growing the batch).
//
// Work decomposition.  For a (sequence b, kv head) pair, the G = Hq/Hkv
// query heads that share it and the T tree nodes form M = G*T query rows that
// all read the same keys, so they are packed as the N dimension of one MFMA
// problem and share every K/V tile staged in LDS.  A workgroup of eight
// waves owns 32*W rows (an "m-tile"; W <= 8 row waves, or 2W waves when each
// row wave takes one 32-key half of every stage) and one slice ("split") of
// the prefix; the other waves only stage K/V;
// the split holding the end of the prefix also takes the T tree keys, with
// the ancestor-or-self mask applied from per-row bitmasks that each lane
// builds from the parent array (kernel argument).  Splits are merged by a
// log-sum-exp combine kernel.  Block ids are remapped so that the m-tiles and
// splits of one (b, kv head) run on the same XCD and share its L2.
//
// Per wave and 32-key sub-block (S^T = K Q^T, then O^T += V^T P^T):
//   - S^T on 32x32 MFMAs: A = K rows (keys) from LDS, B = Q^T from registers
//     (each lane owns one query column);
//   - online softmax per lane in the log2 domain (scores * scale * log2 e),
//     the running max shared with the partner lane (lane ^ 32);
//   - P^T goes straight from the S^T accumulators into the B operand, V^T
//     comes from LDS, where V is stored transposed (and, for bf16, with its
//     4-key groups reordered so each lane reads one 16-byte chunk).
#include <type_traits>

#include "common.h"

namespace medusa {
namespace {

constexpr int kBN = 64;          // keys per LDS stage
constexpr int kMaxWaves = 8;     // waves per workgroup
// Stages of K/V loads in flight (bf16; fp32 stages are twice as large: 1).
constexpr int kPD = 2;
constexpr int kMinChunk = 384;   // smallest prefix split (keys)
constexpr int kTargetWG = kNumCU;   // the launch targets one workgroup per CU

template <typename T, int DH>
struct Cfg {
    static constexpr int KC = Elem<T>::kPer16B;      // elements per 16-byte chunk
    static constexpr int KSTEP = 2 * KC;              // dh per MFMA k-step
    static constexpr int NKS = DH / KSTEP;            // k-steps for q.k
    static constexpr int NDT = DH / 32;               // 32-row dh tiles of O^T
    static constexpr int CPR = DH / KC;               // 16-byte chunks per K row
    static constexpr int KS_STRIDE = DH * (int)sizeof(T) + 16;   // bytes per key row
    static constexpr int VT_STRIDE = kBN * (int)sizeof(T) + 16;  // bytes per dh row
    static constexpr int KS_BYTES = kBN * KS_STRIDE;
    static constexpr int VT_BYTES = DH * VT_STRIDE;
    static constexpr int LDS_BYTES = KS_BYTES + VT_BYTES;
};

struct AttnParams {
    const void *q, *kc, *vc, *kt, *vt;
    const int32_t *prefix_len;
    void *out;
    uint64_t *mask_out;
    float *part_o;      // [nsplit][B][Hq][T][dh]
    float2 *part_ml;    // [nsplit][B][Hq][T]  (max in log2 units, sum)
    int32_t *err;
    int B, Hq, Hkv, Lcap, T, G, M, W, nmt, nsplit, chunk, nwg;
    int ks;             // 1, or 2: waves W..2W-1 take the second 32-key half of every stage
    float c;            // scale * log2(e)
    uint8_t parent[MEDUSA_MAX_TREE];   // parent index; 255 marks the root (never a parent: parent < n <= 255)
};

// position of key k (0..63) of a stage inside a transposed V row
template <typename T>
__device__ __forceinline__ int vt_pos(int k);
template <>
__device__ __forceinline__ int vt_pos<float>(int k) { return k; }
template <>
__device__ __forceinline__ int vt_pos<bf16_t>(int k) {
    // within each 16 keys, 4-key group a goes to 8*(a%2) + 4*(a/2)
    const int a = (k >> 2) & 3;
    return (k & ~15) + 8 * (a & 1) + 4 * (a >> 1) + (k & 3);
}

// Register-staged copy of one 64-key stage (keys [0, nvalid) from kb / vb) to
// LDS: K as rows, V transposed.  load() issues every global load of the
// stage at once (so one memory latency covers the stage and the loads can
// fly while the previous stage is computed); store() writes them to LDS.
// Rows past nvalid are zero: their scores are masked, and zero V keeps
// 0 * garbage out of the sums.  NT = threads of the workgroup.
template <typename T, int DH, int NT>
struct StageCopy {
    using C = Cfg<T, DH>;
    static constexpr int NK = (kBN * C::CPR) / NT;                   // K chunks / thread
    static_assert((kBN * C::CPR) % NT == 0, "K chunks divide evenly over the threads");
    static constexpr int NV = ((kBN / 4) * C::CPR + NT - 1) / NT;    // V units / thread
    // With twice as many threads as V units, the units go to the upper half
    // of the workgroup (waves NW/2 ..): the two waves of a SIMD then start a
    // stage's matrix and vector phases apart, by the transposing stores.
    static constexpr bool kVUpper = (kBN / 4) * C::CPR * 2 == NT;
    __device__ __forceinline__ static int vthread(int tid) { return kVUpper ? tid ^ (NT / 2) : tid; }
    u32x4 k[NK];
    u32x4 v[NV][4];

    // kr / vr cover exactly the stage's valid key rows: rows past them read
    // as zero.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                         int tid) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int ch = tid + i * NT;
            const int key = ch / C::CPR, col = ch % C::CPR;
            k[i] = buf_ld16(kr, (uint32_t)((key * DH + col * C::KC) * (int)sizeof(T)));
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int u = vthread(tid) + i * NT;
            const int kg = u % (kBN / 4), col = u / (kBN / 4);   // see store()
            const bool live = u < (kBN / 4) * C::CPR;   // spare threads: offsets past the
                                                       // range, dropped by the hardware
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[i][j] = buf_ld16(vr, live ? (uint32_t)(((4 * kg + j) * DH + col * C::KC) * (int)sizeof(T))
                                            : 0xFFFFFF00u);
        }
    }

    __device__ __forceinline__ void store(char *lds, int tid) const {
        char *Ks = lds;
        char *Vt = lds + C::KS_BYTES;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int ch = tid + i * NT;
            if (ch < kBN * C::CPR) {
                const int key = ch / C::CPR, col = ch % C::CPR;
                st16(Ks + key * C::KS_STRIDE + col * 16, k[i]);
            }
        }
        // V units: the 16 consecutive threads of a key-group index kg share a
        // column chunk, so each transposed store of 16 lanes fills 16 distinct
        // 4-key slots of one dh row (128 contiguous bytes, no bank conflicts).
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int u = vthread(tid) + i * NT;
            if (u >= (kBN / 4) * C::CPR) continue;
            const int kg = u % (kBN / 4), col = u / (kBN / 4);
            const int pos = vt_pos<T>(4 * kg);
#pragma unroll
            for (int e = 0; e < C::KC; ++e) {
                char *dst = Vt + (col * C::KC + e) * C::VT_STRIDE + pos * (int)sizeof(T);
                if constexpr (sizeof(T) == 2) {
                    // element e of four keys: the low or high halves of word
                    // e/2, paired by byte selects (v_perm_b32: selector bytes
                    // 0-3 pick the second operand's bytes, 4-7 the first's)
                    const int w = e >> 1;
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    const uint32_t lo = __builtin_amdgcn_perm(v[i][1][w], v[i][0][w], sel);
                    const uint32_t hi = __builtin_amdgcn_perm(v[i][3][w], v[i][2][w], sel);
                    *reinterpret_cast<u32x2 *>(dst) = u32x2{lo, hi};
                } else {
                    st16(dst, u32x4{v[i][0][e], v[i][1][e], v[i][2][e], v[i][3][e]});
                }
            }
        }
    }
};

struct RowState {
    float m;      // reference max (log2 units) the block scores are taken
                  // against; -inf before the first key; shared by the lane pair
    float l;      // this lane's part of the softmax denominator
    f32x16 negr;  // bf16: -m in every element (0 while m = -inf), the
                  // accumulator each block's first q.k product starts from
    float thr;    // the block max (relative to m) that moves m: -inf while
                  // m = -inf, then 8 (pipelined kernel)
};

// max over lanes l and l ^ 32 (v_permlane32_swap trades the upper half of
// one operand with the lower half of the other; with both operands x each
// lane then holds x[l] and x[l ^ 32])
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// The first k-step of a 32x32 product, accumulating onto c (not in place).
__device__ __forceinline__ f32x16 mma32_first(const f32x16 &c, const u32x4 &a, const u32x4 &b, bf16_t) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32_first(const f32x16 &c, const u32x4 &a, const u32x4 &b, float) {
    f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c,
                                                      0, 0, 0);
#pragma unroll
    for (int e = 1; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc,
                                                   0, 0, 0);
    return acc;
}

// P^T (the probabilities of one 32-key block, this lane's query) times V^T
// of those keys, accumulated into O^T.  bf16: pk holds them packed in the
// B-operand order of the two 16-key k-steps; fp32: p[16].
template <int DH>
__device__ __forceinline__ void pv_block_bf16(const char *Vt, const u32x4 (&pk)[2],
                                              f32x16 (&o)[Cfg<bf16_t, DH>::NDT], int sub, int h,
                                              int col) {
    using C = Cfg<bf16_t, DH>;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        const char *vrow = Vt + (dt * 32 + col) * C::VT_STRIDE;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(vrow + (sub * 32 + 16 * mm + 8 * h) * 2);
            mma32_step(o[dt], a, pk[mm], bf16_t{});
        }
    }
}
template <int DH>
__device__ __forceinline__ void pv_block_f32(const char *Vt, const float (&p)[16],
                                             f32x16 (&o)[Cfg<float, DH>::NDT], int sub, int h,
                                             int col) {
    using C = Cfg<float, DH>;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        const char *vrow = Vt + (dt * 32 + col) * C::VT_STRIDE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(vrow + (sub * 32 + 8 * i + 4 * h) * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) mma32_f32_single(o[dt], __uint_as_float(a[j]), p[4 * i + j]);
        }
    }
}

// One 64-key stage for one wave (lane: query column col, keys of half h), as
// two 32-key blocks: S^T = K Q^T on the matrix cores, reference update,
// P^T V^T.  Q is pre-scaled by scale * log2(e) and the first product of a
// block accumulates onto -m, so the scores leave the matrix cores already
// in the exponent's frame: p = exp2(s).  masked: apply kind 0 (key < klim)
// or kind 1 (tree ancestor bits of mword); full prefix stages skip masking.
template <typename T, int DH>
__device__ __forceinline__ void attend_stage(const char *lds, const u32x4 (&qf)[Cfg<T, DH>::NKS],
                                             f32x16 (&o)[Cfg<T, DH>::NDT], RowState &st, int lane,
                                             bool masked, int kind, int klim, uint64_t mword,
                                             int sub_lo, int sub_hi) {
    using C = Cfg<T, DH>;
    const char *Ks = lds;
    const char *Vt = lds + C::KS_BYTES;
    const int h = lane >> 5, col = lane & 31;
#pragma unroll 1
    for (int sub = sub_lo; sub < sub_hi; ++sub) {   // 32-key halves of the stage
        const char *krow = Ks + (sub * 32 + col) * C::KS_STRIDE + h * 16;
        f32x16 s;
        if constexpr (sizeof(T) == 2) {
            s = mma32_first(st.negr, *reinterpret_cast<const u32x4 *>(krow), qf[0], T{});
        } else {
            // fp32 keeps no -m tile (its q.k takes more registers): the
            // accumulator starts from -m broadcast on the spot
            const float nr = st.m == -INFINITY ? 0.f : -st.m;
            f32x16 init;
#pragma unroll
            for (int r = 0; r < 16; ++r) init[r] = nr;
            s = mma32_first(init, *reinterpret_cast<const u32x4 *>(krow), qf[0], T{});
        }
#pragma unroll
        for (int ks = 1; ks < C::NKS; ++ks) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(krow + ks * 32);
            mma32_step(s, a, qf[ks], T{});
        }
        // s[r]: key sub*32 + 4h + 8*(r/4) + r%4 of this stage; after one
        // shift by sub*32 + 4h each test uses a constant bit position
        if (masked) {
            const int base = sub * 32 + 4 * h;
            if (kind == 0) {
                const int lim = klim - base;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[r] = 8 * (r >> 2) + (r & 3) < lim ? s[r] : -INFINITY;
            } else {
                const uint32_t bits = (uint32_t)(mword >> base);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[r] = (bits >> (8 * (r >> 2) + (r & 3))) & 1u ? s[r] : -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = pair_max(mx);   // relative to the reference
        // Lazy reference: it only moves when the block max exceeds it by
        // more than 8 (log2 units), so p <= 2^8 and most blocks skip the O
        // rescale; the branch is taken by the whole wave or not at all.  The
        // result does not depend on the reference (exact algebra).
        const bool need = st.m == -INFINITY ? mx > -INFINITY : mx > 8.0f;
        if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
            const float sh = need ? mx : 0.f;
            const float alpha = !need ? 1.f : (st.m == -INFINITY ? 0.f : fast_exp2(-sh));
            st.l *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) o[dt] *= alpha;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] -= sh;
            if (need) st.m = (st.m == -INFINITY ? 0.f : st.m) + sh;
            if constexpr (sizeof(T) == 2) {
                const float nr = st.m == -INFINITY ? 0.f : -st.m;
#pragma unroll
                for (int r = 0; r < 16; ++r) st.negr[r] = nr;
            }
        }
        if constexpr (sizeof(T) == 2) {
            // the probabilities packed to bf16 for the P V product; the row
            // sum takes the same bf16 values (v_dot2 with ones), so the
            // weights of numerator and denominator are the same numbers
            const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
            u32x4 pk[2];
            float acc = st.l;
#pragma unroll
            for (int mm = 0; mm < 2; ++mm)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t v = pack_bf16x2(fast_exp2(s[8 * mm + 2 * w]),
                                                   fast_exp2(s[8 * mm + 2 * w + 1]));
                    pk[mm][w] = v;
                    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v), ones, acc,
                                                          false);
                }
            st.l = acc;
            pv_block_bf16<DH>(Vt, pk, o, sub, h, col);
        } else {
            float p[16];
            float psum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = fast_exp2(s[r]);
                psum += p[r];
            }
            st.l += psum;
            pv_block_f32<DH>(Vt, p, o, sub, h, col);
        }
    }
}

// What a workgroup and each of its lanes own.  Block ids are remapped so
// that the m-tiles and splits of one (b, kv head) run on the same XCD; with
// the key split (ks = 2) waves w and w + W share rows, wave group kgrp taking
// the 32-key half kgrp of every stage.
struct Tile {
    int b, kvh, split, rwave, kgrp, row, t, hq;
    bool rvalid, computes, last;
    int kbeg, kend, nsb;
    uint64_t mw0, mw1, mw2, mw3;   // the lane's ancestor-or-self bits over the tree keys
};

// Work set-up shared by both attention kernels: decodes the block id, loads
// the lane's query row into qf (pre-scaled into the exponent's frame by
// scale * log2 e; bf16: rounded to bf16 once), writes the parent table to
// LDS, records out-of-range prefix lengths (block 0) and the tree mask
// (block 0, when asked), and builds the lane's ancestor bitmask.  Returns
// false when the block's prefix split is empty.  Every thread reaches the
// one barrier inside.
template <typename T, int DH>
__device__ __forceinline__ bool tile_setup(const AttnParams &p, uint8_t *par,
                                           u32x4 (&qf)[Cfg<T, DH>::NKS], Tile &tl) {
    using C = Cfg<T, DH>;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid % kWave, wave = tid / kWave;

    // logical block -> (b, kv head, split, m-tile), m-tile fastest
    const uint32_t lid = xcd_logical_id(blockIdx.x, (uint32_t)p.nwg);
    const int mt = (int)(lid % p.nmt);
    tl.split = (int)((lid / p.nmt) % p.nsplit);
    tl.kvh = (int)((lid / ((uint32_t)p.nmt * p.nsplit)) % p.Hkv);
    tl.b = (int)(lid / ((uint32_t)p.nmt * p.nsplit * p.Hkv));

    // The prefix length, this lane's query row and the parent table are
    // loaded together, before the first wait.  The parent table
    // (kernel-argument bytes) is read into registers first and written to LDS
    // after the query loads are issued: loads complete in order, so waiting
    // for it then does not wait for them.
    static_assert(MEDUSA_MAX_TREE % 4 == 0 && MEDUSA_MAX_TREE / 4 <= 4 * kWave, "parent words");
    const uint32_t parw = tid < MEDUSA_MAX_TREE / 4 ? reinterpret_cast<const uint32_t *>(p.parent)[tid] : 0u;
    const int Lraw = p.prefix_len[tl.b];
    const int col = lane & 31, h = lane >> 5;
    tl.rwave = wave % p.W;
    tl.kgrp = wave / p.W;
    tl.row = mt * 32 * p.W + tl.rwave * 32 + col;
    tl.computes = tl.kgrp < p.ks;
    tl.rvalid = tl.computes && tl.row < p.M;
    const int g = tl.rvalid ? tl.row / p.T : 0;
    tl.t = tl.rvalid ? tl.row % p.T : 0;
    tl.hq = tl.kvh * p.G + g;
    {
        // one resource over the kv head's M query rows (a uniform base: a
        // per-lane resource would need a loop over the distinct lanes);
        // lanes without a row read past its end, which returns 0
        const T *qkv = (const T *)p.q + ((size_t)tl.b * p.Hq + (size_t)tl.kvh * p.G) * p.T * DH;
        const auto qr = make_rsrc(qkv, (uint32_t)((size_t)p.M * DH * sizeof(T)));
        const uint32_t qoff =
            tl.rvalid ? (uint32_t)(((size_t)tl.row * DH + h * C::KC) * sizeof(T)) : 0xFFFFF000u;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
            qf[ks] = buf_ld16(qr, qoff + (uint32_t)(ks * C::KSTEP * sizeof(T)));
    }
    if (tid < MEDUSA_MAX_TREE / 4) reinterpret_cast<uint32_t *>(par)[tid] = parw;

    if (lid == 0 && tid == 0) {
        int bad = 0;
        for (int i = 0; i < p.B; ++i) bad |= (p.prefix_len[i] < 0 || p.prefix_len[i] > p.Lcap);
        *p.err = bad;
    }
    const int L = Lraw < 0 ? 0 : (Lraw > p.Lcap ? p.Lcap : Lraw);
    tl.nsb = L > 0 ? (L + p.chunk - 1) / p.chunk : 1;
    __syncthreads();
    if (p.mask_out && lid == 0) {
        const int W = (p.T + 63) / 64;
        for (int n = tid; n < p.T; n += nthr) {
            uint64_t w[4] = {0ull, 0ull, 0ull, 0ull};
            // walk n, parent(n), ..., root (whose parent entry is 255)
            for (int a = n, guard = 0; guard <= p.T; a = par[a], ++guard) {
                w[a >> 6] |= 1ull << (a & 63);
                if (par[a] == 255) break;
            }
            for (int k = 0; k < W; ++k) p.mask_out[(size_t)n * W + k] = w[k];
        }
    }
    if (tl.split >= tl.nsb) return false;
    tl.kbeg = tl.split * p.chunk;
    tl.kend = tl.kbeg + p.chunk < L ? tl.kbeg + p.chunk : L;
    tl.last = tl.split == tl.nsb - 1;

    uint64_t mw0 = 0, mw1 = 0, mw2 = 0, mw3 = 0;
    for (int a = tl.t, guard = 0; guard <= p.T; a = par[a], ++guard) {
        const uint64_t bit = 1ull << (a & 63);
        const int wi = a >> 6;
        mw0 |= wi == 0 ? bit : 0ull;
        mw1 |= wi == 1 ? bit : 0ull;
        mw2 |= wi == 2 ? bit : 0ull;
        mw3 |= wi == 3 ? bit : 0ull;
        if (par[a] == 255) break;   // a is the root
    }
    tl.mw0 = mw0;
    tl.mw1 = mw1;
    tl.mw2 = mw2;
    tl.mw3 = mw3;

    const float cs = p.c;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t v = qf[ks][w];
            if constexpr (sizeof(T) == 2)
                qf[ks][w] = pack_bf16x2(__uint_as_float(v << 16) * cs,
                                        __uint_as_float(v & 0xFFFF0000u) * cs);
            else
                qf[ks][w] = __float_as_uint(__uint_as_float(v) * cs);
        }
    return true;
}

// The tree ancestor bits of tree-key block wi (64 keys).
__device__ __forceinline__ uint64_t tree_word(const Tile &tl, int wi) {
    return wi == 0 ? tl.mw0 : wi == 1 ? tl.mw1 : wi == 2 ? tl.mw2 : tl.mw3;
}

// Writes this lane's finished O^T columns (nsb == 1: normalised output;
// otherwise fp32 partials with the split's (max, sum)).
template <typename T, int DH>
__device__ __forceinline__ void store_rows(const AttnParams &p, const Tile &tl,
                                           const f32x16 (&o)[Cfg<T, DH>::NDT], float m, float ltot,
                                           int h) {
    using C = Cfg<T, DH>;
    const size_t orow = ((size_t)tl.b * p.Hq + tl.hq) * p.T + tl.t;
    if (tl.nsb == 1) {
        const float inv = 1.0f / ltot;
        T *dst = (T *)p.out + orow * DH;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                T *d4 = dst + dt * 32 + 8 * i + 4 * h;
                if constexpr (sizeof(T) == 2) {
                    const uint32_t lo = pack_bf16x2(o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv);
                    const uint32_t hi = pack_bf16x2(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv);
                    *reinterpret_cast<u32x2 *>(d4) = u32x2{lo, hi};
                } else {
                    *reinterpret_cast<f32x4 *>(d4) =
                        f32x4{o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv, o[dt][4 * i + 2] * inv,
                              o[dt][4 * i + 3] * inv};
                }
            }
    } else {
        const size_t prow = (size_t)tl.split * p.B * p.Hq * p.T + orow;
        float *dst = p.part_o + prow * DH;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4 *>(dst + dt * 32 + 8 * i + 4 * h) =
                    f32x4{o[dt][4 * i], o[dt][4 * i + 1], o[dt][4 * i + 2], o[dt][4 * i + 3]};
        if (h == 0) p.part_ml[prow] = make_float2(m, ltot);
    }
}

// NW waves are launched per workgroup; the first ks * p.W of them own query
// rows (with ks = 2, two waves per row tile, one per 32-key half of each
// stage), all of them share the staging of K/V.
template <typename T, int DH, int NW>
__global__ __launch_bounds__(NW *kWave, 1) void tree_attn_fwd_kernel(AttnParams p) {
    using C = Cfg<T, DH>;
    constexpr int NT = NW * kWave;
    __shared__ __attribute__((aligned(16))) char lds[2][C::LDS_BYTES];   // double buffer
    __shared__ __attribute__((aligned(16))) uint8_t par[MEDUSA_MAX_TREE];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    u32x4 qf[C::NKS];
    Tile tl;
    if (!tile_setup<T, DH>(p, par, qf, tl)) return;
    const int b = tl.b, kvh = tl.kvh, kgrp = tl.kgrp, rwave = tl.rwave;
    const int kbeg = tl.kbeg, kend = tl.kend;
    const bool last = tl.last;
    f32x16 o[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) o[dt] = f32x16{};
    RowState st{-INFINITY, 0.f, f32x16{}, -INFINITY};

    // stages: prefix keys [kbeg, kend) in blocks of kBN, then (last split) the tree keys
    const T *kcb = (const T *)p.kc + ((size_t)b * p.Hkv + kvh) * (size_t)p.Lcap * DH;
    const T *vcb = (const T *)p.vc + ((size_t)b * p.Hkv + kvh) * (size_t)p.Lcap * DH;
    const T *ktb = (const T *)p.kt + ((size_t)b * p.Hkv + kvh) * (size_t)p.T * DH;
    const T *vtb = (const T *)p.vt + ((size_t)b * p.Hkv + kvh) * (size_t)p.T * DH;
    const int npre = (kend - kbeg + kBN - 1) / kBN;
    const int ntree = p.T;        // the lambdas below take no reference to p:
                                  // that would copy the parameter block to scratch
    const int nstage = npre + (last ? (ntree + kBN - 1) / kBN : 0);
    const bool computes = tl.computes;
    const int sub_lo = p.ks == 2 ? kgrp : 0, sub_hi = p.ks == 2 ? kgrp + 1 : 2;

    // PD register sets of staged K/V: the loads of a stage are issued PD
    // stages before it is written to LDS, so PD stages of bytes are in flight
    constexpr int PD = sizeof(T) == 2 ? kPD : 1;   // fp32 stages are twice as large
    StageCopy<T, DH, NT> cp[PD];
    // Stages past the last are issued as empty ranges (their loads return
    // zeros without touching memory), so that every load and store below is
    // unconditional: the compiler then knows exactly how many loads are
    // younger than the ones a store waits for, and keeps PD stages in flight.
    auto issue = [&](StageCopy<T, DH, NT> &dst, int sidx) __attribute__((always_inline)) {
        const T *kb = kcb, *vb = vcb;
        int nv = 0;
        if (sidx < npre) {
            const int k0 = kbeg + sidx * kBN;
            nv = kend - k0 < kBN ? kend - k0 : kBN;
            kb = kcb + (size_t)k0 * DH;
            vb = vcb + (size_t)k0 * DH;
        } else if (sidx < nstage) {
            const int tb = (sidx - npre) * kBN;
            nv = ntree - tb < kBN ? ntree - tb : kBN;
            kb = ktb + (size_t)tb * DH;
            vb = vtb + (size_t)tb * DH;
        }
        const uint32_t nbytes = (uint32_t)(nv * DH * (int)sizeof(T));
        dst.load(make_rsrc(kb, nbytes), make_rsrc(vb, nbytes), tid);
    };
    // Double-buffered LDS stages, one barrier each: stage i+1 (loads issued
    // PD stages earlier) is written to buffer (i+1)%2, free since the last
    // barrier, the loads of stage i+1+PD go out into the register set it
    // freed, and stage i is computed from buffer i%2.  Staging first lets the
    // waves without V units start computing while the others transpose V.
    // The loop is unrolled by PD so that every register set is named
    // statically; it runs a multiple of PD stages, the ones past the last
    // computing nothing.
    // prologue: stages 0 .. PD-1 in flight, stage 0 to LDS, stage PD issued
#pragma unroll
    for (int k = 0; k < PD; ++k) issue(cp[k], k);
    cp[0].store(lds[0], tid);
    issue(cp[0], PD);
    __syncthreads();
    const int nstage_pad = (nstage + PD - 1) / PD * PD;
    for (int base = 0; base < nstage_pad; base += PD) {
#pragma unroll
        for (int k = 0; k < PD; ++k) {   // unrolled: register set (k + 1) % PD is static
            const int sidx = base + k;
            cp[(k + 1) % PD].store(lds[(sidx + 1) & 1], tid);
            issue(cp[(k + 1) % PD], sidx + 1 + PD);
            if (computes && sidx < nstage) {
                int kind = 0, klim = kBN;
                uint64_t mword = 0ull;
                if (sidx < npre) {
                    const int k0 = kbeg + sidx * kBN;
                    klim = kend - k0 < kBN ? kend - k0 : kBN;
                } else {
                    const int wi = sidx - npre;
                    kind = 1;
                    mword = tree_word(tl, wi);
                }
                const bool masked = kind == 1 || klim < kBN;
                attend_stage<T, DH>(lds[sidx & 1], qf, o, st, lane, masked, kind, klim, mword,
                                    sub_lo, sub_hi);
            }
            __syncthreads();
        }
    }

    float ltot = st.l + __shfl_xor(st.l, 32);
    static_assert((C::NDT * 16 + 2) * (kMaxWaves / 2) * kWave * 4 <= 2 * C::LDS_BYTES,
                  "the key-split exchange fits in the stage buffers (W <= kMaxWaves / 2)");
    if (p.ks == 2) {
        // group 1 hands its (max, sum, O) to group 0 through LDS (the stage
        // buffers are free after the loop's last barrier); its max can be
        // -inf (every key of its halves masked), group 0's never is
        float *ob = reinterpret_cast<float *>(&lds[0][0]);
        float2 *mlb = reinterpret_cast<float2 *>(ob + C::NDT * 16 * p.W * kWave);
        const int slot = rwave * kWave + lane;
        if (kgrp == 1) {
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) ob[(dt * 16 + r) * p.W * kWave + slot] = o[dt][r];
            mlb[slot] = make_float2(st.m, ltot);
        }
        __syncthreads();
        if (kgrp != 0) return;
        const float2 ml1 = mlb[slot];
        const float mnew = fmaxf(st.m, ml1.x);
        const float a0 = fast_exp2(st.m - mnew);
        const float a1 = ml1.x == -INFINITY ? 0.f : fast_exp2(ml1.x - mnew);
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o[dt][r] = o[dt][r] * a0 + ob[(dt * 16 + r) * p.W * kWave + slot] * a1;
        ltot = ltot * a0 + ml1.y * a1;
        st.m = mnew;
    }
    if (!tl.rvalid || !computes) return;
    store_rows<T, DH>(p, tl, o, st.m, ltot, lane >> 5);
}

// ---------------------------------------------------------------------------
// Pipelined kernel: bf16, dh = 128, m-tiles of at least five row waves (one
// wave per 32 query rows, each taking both 32-key halves of every stage).
//
// K/V stages go from global memory straight into LDS (16-byte direct loads,
// no staging registers), four stage buffers deep; the loads of stage s + 3
// are issued while stage s is computed.  K and V rows stay key-major.  The
// V^T fragments of the P V product are read with the LDS transpose read
// (ds_read_b64_tr_b16): within each 16 lanes, lane 4r + q addresses four
// consecutive 16-bit elements of row r, and lane i receives element i of the
// four rows, so one read gives a lane four consecutive keys of one dh
// column.  The 16-byte chunks of a row are XOR-swizzled (K: chunk c of key
// row r at slot c ^ (r mod 16); V: at slot c ^ 4 (r mod 4)) so that the
// K fragment reads (16 key rows per 16 lanes, one chunk each) and the
// transpose reads (4 key rows x 64 bytes per 32 lanes) hit distinct banks.
//
// Per wave the 32-key blocks form a pipeline: block j + 1's scores are
// computed on the matrix cores while block j's row max is found (first
// half of the k-steps) and its first 16 keys are exponentiated (second
// half), and the P V product of block j's first 16 keys runs while the
// second 16 are exponentiated.  Blocks past a stage boundary come from the next stage's
// buffer, which the previous barrier made visible; one barrier per stage.
constexpr int kPipeNB = 4;                                     // LDS stage buffers
constexpr int kPipeRB = 128 * 2;                               // bytes per K or V row
constexpr int kPipeOp = kBN * kPipeRB;                         // one operand of one stage
constexpr int kPipeLoads = 2 * (kPipeOp / 1024) / kMaxWaves;   // loads per wave and stage
static_assert(kPipeLoads == 4, "the stage wait below counts four loads per wave");

// instruction classes of the scheduler's group barriers
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgDsRead = 0x100, kSgTrans = 0x400;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// s_waitcnt: at most one stage of this wave's loads (kPipeLoads) still in
// flight, every LDS read returned.  The stage loads are the only vector
// memory operations inside the stage loop.
__device__ __forceinline__ void pipe_wait_stage() { __builtin_amdgcn_s_waitcnt(0x0074); }
__device__ __forceinline__ void pipe_wait_all() { __builtin_amdgcn_s_waitcnt(0x0070); }
// workgroup barrier without memory fences; no memory access moves across it
__device__ __forceinline__ void pipe_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ u32x4 pipe_ld16(const char *lds, uint32_t off) {
    return *reinterpret_cast<const u32x4 *>(lds + off);
}
__device__ __forceinline__ u32x2 pipe_ld_tr(const char *lds, uint32_t off) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_t *)((__attribute__((address_space(3))) char *)lds + off));
    return __builtin_bit_cast(u32x2, v);
}

// The per-lane LDS byte addresses of the fragments (the buffer, half and
// k-step parts are immediate offsets).
struct PipeLane {
    uint32_t ka[8];   // K fragment of k-step ks: key row col, chunk 2 ks + h
    uint32_t va[4];   // V^T transpose read of dh tile dt
};

// One 32-key block.  sc holds its scores against the current reference; the
// next block's scores go to sn (K rows at koff in buffer kbuf); this block's
// V rows are at voff in buffer vbuf.
__device__ __forceinline__ void pipe_block(const char *kbuf, const char *vbuf, uint32_t koff,
                                           uint32_t voff, f32x16 &sc, f32x16 &sn,
                                           const u32x4 (&qf)[8],
                                           f32x16 (&o)[4], RowState &st, const PipeLane &pl,
                                           bool masked, uint32_t bits) {
    if (masked) {   // the same in every lane
        // s[r] is key 4h + 8 (r / 4) + r % 4 of the block; bit k of bits
        // tells whether key 4h + k is visible to this lane's query
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sc[r] = (bits >> (8 * (r >> 2) + (r & 3))) & 1u ? sc[r] : -INFINITY;
    }
    // the next block's scores start from -m (the reference as it is now):
    // its first four k-steps go out before this block's row max, the last
    // four after the reference check, beside this block's exponentials
    // (their K fragments are read now)
    sn = mma32_first(st.negr, pipe_ld16(kbuf, pl.ka[0] + koff), qf[0], bf16_t{});
#pragma unroll
    for (int ks = 1; ks < 4; ++ks) mma32_step(sn, pipe_ld16(kbuf, pl.ka[ks] + koff), qf[ks], bf16_t{});
    u32x4 kr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = pipe_ld16(kbuf, pl.ka[4 + i] + koff);
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = pair_max(mx);
    // issue order up to the reference check: the eight K fragment reads,
    // then each of the first four k-steps followed by four of the row-max
    // operations
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 8, 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 1);
    }
    // lazy reference (as in attend_stage, with the threshold kept in st.thr);
    // a move also applies to the next block's scores, which were taken
    // against the old one
    const bool need = mx > st.thr;
    if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
        const float sh = need ? mx : 0.f;
        const float alpha = !need ? 1.f : (st.m == -INFINITY ? 0.f : fast_exp2(-sh));
        st.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sc[r] -= sh;
            sn[r] -= sh;
        }
        if (need) st.m = (st.m == -INFINITY ? 0.f : st.m) + sh;
        st.thr = st.m == -INFINITY ? -INFINITY : 8.0f;
        const float nr = st.m == -INFINITY ? 0.f : -st.m;
#pragma unroll
        for (int r = 0; r < 16; ++r) st.negr[r] = nr;
    }
    // the rest of the next block's k-steps (a reference move above applied
    // to the part already summed, which the rest adds to unchanged)
#pragma unroll
    for (int ks = 4; ks < 8; ++ks) mma32_step(sn, kr[ks - 4], qf[ks], bf16_t{});
    // probabilities packed to bf16 for the P V product (k-step mm: keys
    // 16 mm + 4h + 8 (e / 4) + e % 4 in element e of the B operand); the row
    // sum takes the same bf16 values
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float acc = st.l;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
        u32x4 pk;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t v = pack_bf16x2(fast_exp2(sc[8 * mm + 2 * w]), fast_exp2(sc[8 * mm + 2 * w + 1]));
            pk[w] = v;
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v), ones, acc, false);
        }
        // A operand: V^T rows 32 dt + col; elements 0-3 keys 16 mm + 4h + 0..3,
        // elements 4-7 keys 16 mm + 4h + 8..11 (two transpose reads)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const u32x2 a0 = pipe_ld_tr(vbuf, pl.va[dt] + voff + (uint32_t)(16 * mm) * kPipeRB);
            const u32x2 a1 = pipe_ld_tr(vbuf, pl.va[dt] + voff + (uint32_t)(16 * mm + 8) * kPipeRB);
            mma32_step(o[dt], u32x4{a0[0], a0[1], a1[0], a1[1]}, pk, bf16_t{});
        }
    }
    st.l = acc;
    // issue order after the reference check:
    //   the V^T reads of keys 0-15;
    //   the last four k-steps of the next block's scores, each followed by
    //   two exponentials of keys 0-15;
    //   the V^T reads of keys 16-31;
    //   the four P V products of keys 0-15, each followed by two
    //   exponentials of keys 16-31;
    //   the four P V products of keys 16-31.
    // Left to itself the compiler issues each group of matrix products back
    // to back and the exponentials only after them, so that the matrix
    // cores wait on this wave's exponentials.
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgTrans, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 8, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgTrans, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 4, 0);
}

// The four stage buffers, K and V (16 KiB each), as separate LDS variables
// named by compile-time index only: the compiler then tells a read of one
// buffer from a direct load into another, and adds no wait for loads still
// landing elsewhere.  (Only the pipelined kernel uses them.)
__shared__ __attribute__((aligned(1024))) char pipe_k0[kPipeOp], pipe_k1[kPipeOp], pipe_k2[kPipeOp],
    pipe_k3[kPipeOp];
__shared__ __attribute__((aligned(1024))) char pipe_v0[kPipeOp], pipe_v1[kPipeOp], pipe_v2[kPipeOp],
    pipe_v3[kPipeOp];
template <int B>
__device__ __forceinline__ char *pipe_kbuf() {
    if constexpr (B == 0) return pipe_k0;
    else if constexpr (B == 1) return pipe_k1;
    else if constexpr (B == 2) return pipe_k2;
    else return pipe_k3;
}
template <int B>
__device__ __forceinline__ char *pipe_vbuf() {
    if constexpr (B == 0) return pipe_v0;
    else if constexpr (B == 1) return pipe_v1;
    else if constexpr (B == 2) return pipe_v2;
    else return pipe_v3;
}

// Both blocks of one stage held in buffer B (the second block's successor
// is the first block of the next stage, in buffer B + 1).  The scores
// alternate between sc and sn, so after a stage the current ones are in sc
// again.  masked (the same in every lane): apply vis, whose bit k is set
// when key k of the stage is visible to this lane's query.
template <int B>
__device__ __forceinline__ void pipe_stage(f32x16 &sc, f32x16 &sn,
                                           const u32x4 (&qf)[8], f32x16 (&o)[4], RowState &st,
                                           const PipeLane &pl, int h, bool masked, uint64_t vis) {
    const char *kc = pipe_kbuf<B>(), *vc = pipe_vbuf<B>();
    const char *kn = pipe_kbuf<(B + 1) & (kPipeNB - 1)>();
    // The V buffers lie past the reach of the 16-bit read offset, so each
    // stage forms its own four V addresses; the empty asm hides the lane
    // offsets' origin, which keeps the compiler from holding all sixteen
    // (buffer, dh tile) addresses in registers across the loop.
    PipeLane ps = pl;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) asm volatile("" : "+v"(ps.va[dt]));
    pipe_block(kc, vc, kPipeOp / 2, 0, sc, sn, qf, o, st, ps, masked, (uint32_t)(vis >> (4 * h)));
    pipe_block(kn, vc, 0, kPipeOp / 2, sn, sc, qf, o, st, ps, masked, (uint32_t)(vis >> (32 + 4 * h)));
}

// Where a workgroup's stages come from, and this wave's share of their loads.
struct PipeSrc {
    const char *kcb, *vcb, *ktb, *vtb;   // prefix K/V and tree K/V rows of (b, kv head)
    int kbeg, kend, npre, nstage, ntree;
    int wave;
    uint32_t ok0, ok1, ov0, ov1;         // byte offsets of this lane's loads within a stage
};

// Stage sidx into buffer B.  The wave issues instructions j = wave and
// wave + 8 of each operand, each moving key rows 4 j .. 4 j + 3 (lane l: row
// 4 j + l / 16, LDS slot l % 16, which holds chunk slot ^ swizzle(row)).  The
// loads go through a buffer resource covering the stage's keys only, so
// rows past them read as zeros (their scores are masked; zero V rows add
// nothing), and the lane offsets stay the same for every stage.  Stages past
// the last load the last one again, into a buffer nothing reads, so that
// every stage issues the same loads.
template <int B>
__device__ __forceinline__ void pipe_issue(const PipeSrc &ps, int sidx) {
    char *dk = pipe_kbuf<B>(), *dv = pipe_vbuf<B>();
    const int se = sidx < ps.nstage ? sidx : ps.nstage - 1;
    const char *kb, *vb;
    int nv;
    if (se < ps.npre) {
        const int k0 = ps.kbeg + se * kBN;
        nv = ps.kend - k0 < kBN ? ps.kend - k0 : kBN;
        kb = ps.kcb + (size_t)k0 * kPipeRB;
        vb = ps.vcb + (size_t)k0 * kPipeRB;
    } else {
        const int tb = (se - ps.npre) * kBN;
        nv = ps.ntree - tb < kBN ? ps.ntree - tb : kBN;
        kb = ps.ktb + (size_t)tb * kPipeRB;
        vb = ps.vtb + (size_t)tb * kPipeRB;
    }
    const uint32_t nbytes = (uint32_t)nv * kPipeRB;
    const auto kr = make_rsrc(kb, nbytes), vr = make_rsrc(vb, nbytes);
    typedef __attribute__((address_space(3))) void *lds_vptr_t;
    const uint32_t d0 = (uint32_t)ps.wave * 1024u, d1 = (uint32_t)(ps.wave + 8) * 1024u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_vptr_t)(dk + d0), 16, ps.ok0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_vptr_t)(dv + d0), 16, ps.ov0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_vptr_t)(dk + d1), 16, ps.ok1, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_vptr_t)(dv + d1), 16, ps.ov1, 0, 0, 0);
}

// One pipeline step: stage sidx from buffer B.  Loads of stage sidx + 3 go
// out, both blocks are computed (the prefix tail and the tree stages with
// vis applied), the wave waits for its loads of stage sidx + 2, barrier.
template <int B>
__device__ __forceinline__ void pipe_step(const PipeSrc &ps, int sidx, bool computes, int nfull,
                                          uint64_t tw0, uint64_t tw1, uint64_t tw2, uint64_t tw3,
                                          f32x16 &sc, f32x16 &sn, const u32x4 (&qf)[8],
                                          f32x16 (&o)[4], RowState &st, const PipeLane &pl, int h) {
    pipe_issue<(B + 3) & (kPipeNB - 1)>(ps, sidx + 3);
    if (computes) {
        // the prefix tail: its first klim (< 64) keys; a tree stage: the
        // lane's ancestor-or-self bits
        const bool masked = sidx >= nfull;
        uint64_t vis = 0ull;
        if (masked) {   // the same in every lane
            const int klim = ps.kend - (ps.kbeg + sidx * kBN);
            const int wi = sidx - ps.npre;
            const uint64_t tw = wi <= 0 ? tw0 : wi == 1 ? tw1 : wi == 2 ? tw2 : tw3;
            vis = sidx < ps.npre ? (1ull << klim) - 1ull : tw;
        }
        pipe_stage<B>(sc, sn, qf, o, st, pl, h, masked, vis);
    }
    pipe_wait_stage();
    pipe_barrier();
}

__global__ __launch_bounds__(kMaxWaves *kWave, 1) void tree_attn_pipe_kernel(AttnParams p) {
    using T = bf16_t;
    constexpr int DH = 128;
    __shared__ __attribute__((aligned(16))) uint8_t par[MEDUSA_MAX_TREE];

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    u32x4 qf[8];
    Tile tl;
    if (!tile_setup<T, DH>(p, par, qf, tl)) return;
    const bool computes = tl.computes;
    const int col = lane & 31, h = lane >> 5;

    PipeSrc ps;
    {
        const size_t bh = (size_t)tl.b * p.Hkv + tl.kvh;
        ps.kcb = (const char *)p.kc + bh * (size_t)p.Lcap * kPipeRB;
        ps.vcb = (const char *)p.vc + bh * (size_t)p.Lcap * kPipeRB;
        ps.ktb = (const char *)p.kt + bh * (size_t)p.T * kPipeRB;
        ps.vtb = (const char *)p.vt + bh * (size_t)p.T * kPipeRB;
        ps.kbeg = tl.kbeg;
        ps.kend = tl.kend;
        ps.ntree = p.T;
        ps.npre = (tl.kend - tl.kbeg + kBN - 1) / kBN;
        ps.nstage = ps.npre + (tl.last ? (p.T + kBN - 1) / kBN : 0);
        ps.wave = wave;
        const int row0 = 4 * wave + (lane >> 4), row1 = row0 + 32;
        const uint32_t cv = (uint32_t)(((lane & 15) ^ (4 * (lane >> 4))) * 16);
        ps.ok0 = (uint32_t)(row0 * kPipeRB + ((lane & 15) ^ (row0 & 15)) * 16);
        ps.ok1 = (uint32_t)(row1 * kPipeRB + ((lane & 15) ^ (row1 & 15)) * 16);
        ps.ov0 = (uint32_t)row0 * kPipeRB + cv;
        ps.ov1 = (uint32_t)row1 * kPipeRB + cv;
    }
    const int nfull = (tl.kend - tl.kbeg) / kBN;   // prefix stages with all 64 keys (no mask)
    const int nstage = ps.nstage;
    const uint64_t tw0 = tl.mw0, tw1 = tl.mw1, tw2 = tl.mw2, tw3 = tl.mw3;

    PipeLane pl;
    {
        const uint32_t ky = (uint32_t)(h ^ (col & 15));
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) pl.ka[ks] = (uint32_t)col * kPipeRB + ((32u * ks) ^ (16u * ky));
        const int r4 = (lane >> 2) & 3, q = lane & 3, gm = (lane >> 4) & 1;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            pl.va[dt] = (uint32_t)((4 * h + r4) * kPipeRB + (2 * gm + (q >> 1)) * 16 + (q & 1) * 8 +
                                   64 * (dt ^ r4));
    }

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    RowState st{-INFINITY, 0.f, f32x16{}, -INFINITY};
    f32x16 sc = f32x16{}, sn = f32x16{};

    // block 0 (first 32 keys of stage 0) before the pipeline starts
    pipe_issue<0>(ps, 0);
    pipe_issue<1>(ps, 1);
    pipe_issue<2>(ps, 2);
    pipe_wait_stage();   // stages 0 and 1: this wave's loads
    pipe_barrier();      // ... and every wave's
    if (computes) {
        sc = mma32_first(st.negr, pipe_ld16(pipe_k0, pl.ka[0]), qf[0], bf16_t{});
#pragma unroll
        for (int ks = 1; ks < 8; ++ks) mma32_step(sc, pipe_ld16(pipe_k0, pl.ka[ks]), qf[ks], bf16_t{});
    }
    // stage s in buffer s mod 4, named statically: the loop is unrolled by four
    for (int s = 0; s < nstage; s += kPipeNB) {
        pipe_step<0>(ps, s, computes, nfull, tw0, tw1, tw2, tw3, sc, sn, qf, o, st, pl, h);
        if (s + 1 >= nstage) break;
        pipe_step<1>(ps, s + 1, computes, nfull, tw0, tw1, tw2, tw3, sc, sn, qf, o, st, pl, h);
        if (s + 2 >= nstage) break;
        pipe_step<2>(ps, s + 2, computes, nfull, tw0, tw1, tw2, tw3, sc, sn, qf, o, st, pl, h);
        if (s + 3 >= nstage) break;
        pipe_step<3>(ps, s + 3, computes, nfull, tw0, tw1, tw2, tw3, sc, sn, qf, o, st, pl, h);
    }
    pipe_wait_all();   // the loads past the last stage are still writing LDS

    const float ltot = st.l + __shfl_xor(st.l, 32);
    if (!tl.rvalid) return;
    store_rows<T, DH>(p, tl, o, st.m, ltot, h);
}

// Merge split partials of the rows whose prefix used more than one split:
// one wave per row; lane j holds split j's (max, sum).  Up to kCombU splits
// every load goes out in one round; past that, 64 splits' (max, sum) per
// round, then the O partials with kCombU splits of loads in flight.
constexpr int kCombU = 8;
template <typename T, int DH>
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(AttnParams p) {
    const int lane = threadIdx.x % kWave;
    const size_t rowid = (size_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const size_t nrows = (size_t)p.B * p.Hq * p.T;
    if (rowid >= nrows) return;
    const int b = (int)(rowid / ((size_t)p.Hq * p.T));
    constexpr int PER = DH / kWave;
    if (p.nsplit <= kCombU) {
        // One round of loads: the prefix length, every split's (max, sum)
        // (lane j: split j) and O partials are all issued before any wait.
        // Splits past the row's own count were never written: they are
        // skipped, not weighted by zero (their bytes may be NaN).
        const int j = lane < p.nsplit ? lane : 0;
        const float2 ml = p.part_ml[(size_t)j * nrows + rowid];
        float v[kCombU][PER];
#pragma unroll
        for (int u = 0; u < kCombU; ++u) {
            if (u < p.nsplit) {   // the same in every lane; v[u] is read only for u < nsb
                const float *src = p.part_o + ((size_t)u * nrows + rowid) * DH + lane * PER;
#pragma unroll
                for (int e = 0; e < PER; ++e) v[u][e] = src[e];
            }
        }
        int L = p.prefix_len[b];
        L = L < 0 ? 0 : (L > p.Lcap ? p.Lcap : L);
        const int nsb = L > 0 ? (L + p.chunk - 1) / p.chunk : 1;
        if (nsb == 1) return;
        const bool live = lane < nsb;
        float mmax = live ? ml.x : -INFINITY;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, m));
        const float w = live ? fast_exp2(ml.x - mmax) : 0.f;
        float den = live ? w * ml.y : 0.f;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) den += __shfl_xor(den, m);
        float acc[PER] = {};
#pragma unroll
        for (int u = 0; u < kCombU; ++u) {
            const float wu = __shfl(w, u);
            if (u < nsb) {   // the same in every lane
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] += wu * v[u][e];
            }
        }
        const float inv = 1.0f / den;
        T *dst = (T *)p.out + rowid * DH;
#pragma unroll
        for (int e = 0; e < PER; ++e) dst[lane * PER + e] = Elem<T>::from_f32(acc[e] * inv);
        return;
    }
    int L = p.prefix_len[b];
    L = L < 0 ? 0 : (L > p.Lcap ? p.Lcap : L);
    const int nsb = L > 0 ? (L + p.chunk - 1) / p.chunk : 1;
    if (nsb == 1) return;
    float mmax = -INFINITY;
    for (int s0 = 0; s0 < nsb; s0 += kWave) {
        const float m = s0 + lane < nsb ? p.part_ml[(size_t)(s0 + lane) * nrows + rowid].x : -INFINITY;
        mmax = fmaxf(mmax, m);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, m));
    float acc[PER] = {};
    float den = 0.f;
    for (int s0 = 0; s0 < nsb; s0 += kWave) {
        float w = 0.f;
        if (s0 + lane < nsb) {
            const float2 ml = p.part_ml[(size_t)(s0 + lane) * nrows + rowid];
            w = fast_exp2(ml.x - mmax);
            den += w * ml.y;
        }
        const int n = nsb - s0 < kWave ? nsb - s0 : kWave;
        for (int j0 = 0; j0 < n; j0 += kCombU) {
            float v[kCombU][PER];
#pragma unroll
            for (int u = 0; u < kCombU; ++u) {
                const int sp = s0 + (j0 + u < n ? j0 + u : n - 1);   // clamped: weight 0 below
                const float *src = p.part_o + ((size_t)sp * nrows + rowid) * DH + lane * PER;
#pragma unroll
                for (int e = 0; e < PER; ++e) v[u][e] = src[e];
            }
#pragma unroll
            for (int u = 0; u < kCombU; ++u) {
                const float wu = __shfl(w, j0 + u < n ? j0 + u : 0);
                const float wj = j0 + u < n ? wu : 0.f;
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] += wj * v[u][e];
            }
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) den += __shfl_xor(den, m);
    const float inv = 1.0f / den;
    T *dst = (T *)p.out + rowid * DH;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[lane * PER + e] = Elem<T>::from_f32(acc[e] * inv);
}

// The same merge for up to kCombU splits with two rows per wave (lanes
// 0-31 and 32-63), each lane holding DH / 32 elements of its row (16 bytes
// of an fp32 partial per split at dh = 128): half the load instructions of
// one row per wave.  One round of loads as above; the (max, sum) of a row's
// split j sits in lane j of its half, and every reduction stays within the
// half.
template <typename T, int DH>
__global__ __launch_bounds__(256) void tree_attn_combine2_kernel(AttnParams p) {
    const int lane = threadIdx.x % kWave, hl = lane % 32, half = lane / 32;
    const size_t nrows = (size_t)p.B * p.Hq * p.T;
    const size_t row = ((size_t)blockIdx.x * 4 + threadIdx.x / kWave) * 2 + half;
    const bool rv = row < nrows;
    const size_t rid = rv ? row : nrows - 1;   // a missing second row: a copy, never stored
    const int b = (int)(rid / ((size_t)p.Hq * p.T));
    constexpr int PER = DH / 32;
    const int j = hl < p.nsplit ? hl : 0;
    const float2 ml = p.part_ml[(size_t)j * nrows + rid];
    float v[kCombU][PER];
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
        if (u < p.nsplit) {   // the same in every lane; v[u] is read only for u < nsb
            const float *src = p.part_o + ((size_t)u * nrows + rid) * DH + hl * PER;
#pragma unroll
            for (int e = 0; e < PER; ++e) v[u][e] = src[e];
        }
    }
    int L = p.prefix_len[b];
    L = L < 0 ? 0 : (L > p.Lcap ? p.Lcap : L);
    const int nsb = L > 0 ? (L + p.chunk - 1) / p.chunk : 1;   // at most nsplit
    const bool live = hl < nsb;
    float mmax = live ? ml.x : -INFINITY;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, m));
    const float w = live ? fast_exp2(ml.x - mmax) : 0.f;
    float den = live ? w * ml.y : 0.f;
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) den += __shfl_xor(den, m);
    float acc[PER] = {};
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
        const float wu = __shfl(w, half * 32 + u);
        if (u < nsb) {
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += wu * v[u][e];
        }
    }
    if (!rv || nsb == 1) return;   // one split: the main kernel wrote the row
    const float inv = 1.0f / den;
    T *dst = (T *)p.out + rid * DH + hl * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = Elem<T>::from_f32(acc[e] * inv);
}

struct AttnPlan {
    int G, M, W, nmt, ks, nsplit, chunk, nwg;
    size_t err_off, o_off, ml_off, total;
};

AttnPlan attn_plan(int B, int Hq, int Hkv, int Lcap, int dh, int T, int dtype) {
    AttnPlan P;
    P.G = Hq / Hkv;
    P.M = P.G * T;
    const int waves = (P.M + 31) / 32;
    P.W = waves < kMaxWaves ? waves : kMaxWaves;
    P.nmt = (P.M + 32 * P.W - 1) / (32 * P.W);
    // few row waves: a second wave group takes the other key half of each stage
    P.ks = P.W <= kMaxWaves / 2 ? 2 : 1;
    const long long base = (long long)B * Hkv * P.nmt;
    int want = (int)((kTargetWG + base - 1) / base);
    // each split writes M rows of fp32 partials: with many rows per kv head
    // keep splits long so that the partials stay small next to the K/V bytes
    const int min_chunk = P.M > 128 ? 2 * kMinChunk : kMinChunk;
    const int cap = Lcap > 0 ? (Lcap + min_chunk - 1) / min_chunk : 1;
    want = want < 1 ? 1 : (want > cap ? cap : want);
    if (Lcap <= 0) {
        P.chunk = kBN;
        P.nsplit = 1;
    } else {
        int ch = (Lcap + want - 1) / want;
        ch = (ch + kBN - 1) / kBN * kBN;
        P.chunk = ch;
        P.nsplit = (Lcap + ch - 1) / ch;
    }
    // grids past the launch limits (one-dimensional grids of at most
    // 2^31 - 1 workgroups; the combine's eight rows per workgroup) are
    // rejected by the caller: nwg = -1
    const long long nwg = base * P.nsplit;
    const long long nrows = (long long)B * Hq * T;
    P.nwg = nwg <= 0x7FFFFFFFLL && (nrows + 7) / 8 <= 0x7FFFFFFFLL ? (int)nwg : -1;
    const size_t rows = (size_t)B * Hq * T;
    P.err_off = 0;
    P.o_off = 256;
    const size_t osz = P.nsplit > 1 ? (size_t)P.nsplit * rows * dh * sizeof(float) : 0;
    P.ml_off = P.o_off + align_up(osz, 256);
    const size_t mlsz = P.nsplit > 1 ? (size_t)P.nsplit * rows * sizeof(float2) : 0;
    P.total = P.ml_off + align_up(mlsz, 256);
    (void)dtype;
    return P;
}

int check_tree(const int32_t *parent, int T) {
    if (!parent) return MEDUSA_ERR_NULL;
    if (T < 1 || T > MEDUSA_MAX_TREE) return MEDUSA_ERR_SHAPE;
    if (parent[0] != -1) return MEDUSA_ERR_TREE;
    for (int n = 1; n < T; ++n)
        if (parent[n] < 0 || parent[n] >= n) return MEDUSA_ERR_TREE;
    return MEDUSA_OK;
}

int check_attn(const void *q, const void *kc, const void *vc, const int32_t *pl, const void *kt,
               const void *vt, const int32_t *parent, int B, int Hq, int Hkv, int Lcap, int dh,
               int T, float scale, int dtype, const void *out) {
    if (!q || !kc || !vc || !pl || !kt || !vt || !out) return MEDUSA_ERR_NULL;
    if (dtype != MEDUSA_F32 && dtype != MEDUSA_BF16) return MEDUSA_ERR_DTYPE;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Lcap < 0 || (dh != 64 && dh != 128) ||
        T < 1 || T > MEDUSA_MAX_TREE)
        return MEDUSA_ERR_SHAPE;
    if ((long long)B * Hkv * Lcap * dh >= (1LL << 40)) return MEDUSA_ERR_SHAPE;
    // the query rows of one kv head are read through one buffer resource
    if ((long long)(Hq / Hkv) * T * dh * (dtype == MEDUSA_BF16 ? 2 : 4) >= (1LL << 32))
        return MEDUSA_ERR_SHAPE;
    if (!(scale > 0.f) || scale != scale || scale == INFINITY) return MEDUSA_ERR_PARAM;
    return check_tree(parent, T);
}

template <typename T, int DH>
int launch_attn(const AttnParams &p, hipStream_t st) {
    // Eight waves (two per SIMD at <= 256 registers each): with few row
    // waves (ks * W <= 4) the others only stage K/V, which measured faster
    // than four waves at one per SIMD.
    // bf16 with dh = 128 and every wave owning rows: the pipelined kernel
    if (sizeof(T) == 2 && DH == 128 && p.ks == 1)
        hipLaunchKernelGGL(tree_attn_pipe_kernel, dim3(p.nwg), dim3(kMaxWaves * kWave), 0, st, p);
    else
        hipLaunchKernelGGL((tree_attn_fwd_kernel<T, DH, kMaxWaves>), dim3(p.nwg),
                           dim3(kMaxWaves * kWave), 0, st, p);
    if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    if (p.nsplit > 1) {
        const size_t rows = (size_t)p.B * p.Hq * p.T;
        if (p.nsplit <= kCombU)
            hipLaunchKernelGGL((tree_attn_combine2_kernel<T, DH>), dim3((unsigned)((rows + 7) / 8)),
                               dim3(256), 0, st, p);
        else
            hipLaunchKernelGGL((tree_attn_combine_kernel<T, DH>), dim3((unsigned)((rows + 3) / 4)),
                               dim3(256), 0, st, p);
        if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    }
    return MEDUSA_OK;
}

}  // namespace
}  // namespace medusa

using namespace medusa;

extern "C" size_t tree_attention_workspace_bytes(int B, int Hq, int Hkv, int Lcap, int dh, int T,
                                                 int dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Lcap < 0 || (dh != 64 && dh != 128) ||
        T < 1 || T > MEDUSA_MAX_TREE || (dtype != MEDUSA_F32 && dtype != MEDUSA_BF16))
        return 0;
    if ((long long)(Hq / Hkv) * T * dh * (dtype == MEDUSA_BF16 ? 2 : 4) >= (1LL << 32)) return 0;
    const AttnPlan P = attn_plan(B, Hq, Hkv, Lcap, dh, T, dtype);
    return P.nwg < 0 ? 0 : P.total;
}

extern "C" int tree_attention(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *prefix_len, const void *k_tree, const void *v_tree,
                              const int32_t *parent, int B, int Hq, int Hkv, int Lcap, int dh,
                              int T, float scale, int dtype, void *out, uint64_t *mask_out,
                              void *ws, size_t ws_bytes, void *stream) {
    int st = check_attn(q, k_cache, v_cache, prefix_len, k_tree, v_tree, parent, B, Hq, Hkv, Lcap,
                        dh, T, scale, dtype, out);
    if (st != MEDUSA_OK) return st;
    const AttnPlan P = attn_plan(B, Hq, Hkv, Lcap, dh, T, dtype);
    if (P.nwg < 0) return MEDUSA_ERR_SHAPE;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < P.total) return MEDUSA_ERR_WORKSPACE;
    AttnParams p;
    p.q = q;
    p.kc = k_cache;
    p.vc = v_cache;
    p.kt = k_tree;
    p.vt = v_tree;
    p.prefix_len = prefix_len;
    p.out = out;
    p.mask_out = mask_out;
    p.err = (int32_t *)((char *)ws + P.err_off);
    p.part_o = (float *)((char *)ws + P.o_off);
    p.part_ml = (float2 *)((char *)ws + P.ml_off);
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Lcap = Lcap;
    p.T = T;
    p.G = P.G;
    p.M = P.M;
    p.W = P.W;
    p.ks = P.ks;
    p.nmt = P.nmt;
    p.nsplit = P.nsplit;
    p.chunk = P.chunk;
    p.nwg = P.nwg;
    p.c = scale * 1.4426950408889634f;
    for (int i = 0; i < MEDUSA_MAX_TREE; ++i)
        p.parent[i] = i < T && parent[i] >= 0 ? (uint8_t)parent[i] : (uint8_t)255;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == MEDUSA_BF16)
        return dh == 128 ? launch_attn<bf16_t, 128>(p, s) : launch_attn<bf16_t, 64>(p, s);
    return dh == 128 ? launch_attn<float, 128>(p, s) : launch_attn<float, 64>(p, s);
}
