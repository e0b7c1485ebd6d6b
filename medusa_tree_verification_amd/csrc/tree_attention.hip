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

// NW waves are launched per workgroup; the first ks * p.W of them own query
// rows (with ks = 2, two waves per row tile, one per 32-key half of each
// stage), all of them share the staging of K/V.
template <typename T, int DH, int NW>
__global__ __launch_bounds__(NW *kWave, 1) void tree_attn_fwd_kernel(AttnParams p) {
    using C = Cfg<T, DH>;
    constexpr int NT = NW * kWave;
    __shared__ __attribute__((aligned(16))) char lds[2][C::LDS_BYTES];   // double buffer
    __shared__ __attribute__((aligned(16))) uint8_t par[MEDUSA_MAX_TREE];

    const int tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid % kWave, wave = tid / kWave;

    // logical block -> (b, kv head, split, m-tile), m-tile fastest
    const uint32_t lid = xcd_logical_id(blockIdx.x, (uint32_t)p.nwg);
    const int mt = (int)(lid % p.nmt);
    const int split = (int)((lid / p.nmt) % p.nsplit);
    const int kvh = (int)((lid / ((uint32_t)p.nmt * p.nsplit)) % p.Hkv);
    const int b = (int)(lid / ((uint32_t)p.nmt * p.nsplit * p.Hkv));

    // The prefix length, this lane's query row and the parent table are
    // loaded together, before the first wait.  The parent table
    // (kernel-argument bytes) is read into registers first and written to LDS
    // after the query loads are issued: loads complete in order, so waiting
    // for it then does not wait for them.
    static_assert(MEDUSA_MAX_TREE % 4 == 0 && MEDUSA_MAX_TREE / 4 <= 4 * kWave, "parent words");
    const uint32_t parw = tid < MEDUSA_MAX_TREE / 4 ? reinterpret_cast<const uint32_t *>(p.parent)[tid] : 0u;
    const int Lraw = p.prefix_len[b];
    const int col = lane & 31, h = lane >> 5;
    // with the key split, waves w and w + W share rows: wave group kgrp takes
    // the 32-key half kgrp of every stage
    const int rwave = wave % p.W, kgrp = wave / p.W;
    const int row = mt * 32 * p.W + rwave * 32 + col;
    const bool rvalid = kgrp < p.ks && row < p.M;
    const int g = rvalid ? row / p.T : 0;
    const int t = rvalid ? row % p.T : 0;
    const int hq = kvh * p.G + g;
    u32x4 qf[C::NKS];
    {
        // one resource over the kv head's M query rows (a uniform base: a
        // per-lane resource would need a loop over the distinct lanes);
        // lanes without a row read past its end, which returns 0
        const T *qkv = (const T *)p.q + ((size_t)b * p.Hq + (size_t)kvh * p.G) * p.T * DH;
        const auto qr = make_rsrc(qkv, (uint32_t)((size_t)p.M * DH * sizeof(T)));
        const uint32_t qoff = rvalid ? (uint32_t)(((size_t)row * DH + h * C::KC) * sizeof(T)) : 0xFFFFF000u;
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
    const int nsb = L > 0 ? (L + p.chunk - 1) / p.chunk : 1;
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
    if (split >= nsb) return;
    const int kbeg = split * p.chunk;
    const int kend = kbeg + p.chunk < L ? kbeg + p.chunk : L;
    const bool last = split == nsb - 1;

    uint64_t mw0 = 0, mw1 = 0, mw2 = 0, mw3 = 0;
    for (int a = t, guard = 0; guard <= p.T; a = par[a], ++guard) {
        const uint64_t bit = 1ull << (a & 63);
        const int wi = a >> 6;
        mw0 |= wi == 0 ? bit : 0ull;
        mw1 |= wi == 1 ? bit : 0ull;
        mw2 |= wi == 2 ? bit : 0ull;
        mw3 |= wi == 3 ? bit : 0ull;
        if (par[a] == 255) break;   // a is the root
    }

    // Q pre-scaled into the exponent's frame, scale * log2(e) (bf16: rounded
    // to bf16 once)
    {
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
    }
    f32x16 o[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) o[dt] = f32x16{};
    RowState st{-INFINITY, 0.f, f32x16{}};

    // stages: prefix keys [kbeg, kend) in blocks of kBN, then (last split) the tree keys
    const T *kcb = (const T *)p.kc + ((size_t)b * p.Hkv + kvh) * (size_t)p.Lcap * DH;
    const T *vcb = (const T *)p.vc + ((size_t)b * p.Hkv + kvh) * (size_t)p.Lcap * DH;
    const T *ktb = (const T *)p.kt + ((size_t)b * p.Hkv + kvh) * (size_t)p.T * DH;
    const T *vtb = (const T *)p.vt + ((size_t)b * p.Hkv + kvh) * (size_t)p.T * DH;
    const int npre = (kend - kbeg + kBN - 1) / kBN;
    const int ntree = p.T;        // the lambdas below take no reference to p:
                                  // that would copy the parameter block to scratch
    const int nstage = npre + (last ? (ntree + kBN - 1) / kBN : 0);
    const bool computes = kgrp < p.ks;
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
                    mword = wi == 0 ? mw0 : wi == 1 ? mw1 : wi == 2 ? mw2 : mw3;
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
    if (!rvalid || !computes) return;
    const size_t orow = ((size_t)b * p.Hq + hq) * p.T + t;
    if (nsb == 1) {
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
        const size_t prow = (size_t)split * p.B * p.Hq * p.T + orow;
        float *dst = p.part_o + prow * DH;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4 *>(dst + dt * 32 + 8 * i + 4 * h) =
                    f32x4{o[dt][4 * i], o[dt][4 * i + 1], o[dt][4 * i + 2], o[dt][4 * i + 3]};
        if (h == 0) p.part_ml[prow] = make_float2(st.m, ltot);
    }
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
    P.nwg = (int)(base * P.nsplit);
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
    if (!(scale > 0.f) || scale != scale || scale == INFINITY) return MEDUSA_ERR_PARAM;
    return check_tree(parent, T);
}

template <typename T, int DH>
int launch_attn(const AttnParams &p, hipStream_t st) {
    // Eight waves (two per SIMD at <= 256 registers each): with few row
    // waves (ks * W <= 4) the others only stage K/V, which measured faster
    // than four waves at one per SIMD.
    hipLaunchKernelGGL((tree_attn_fwd_kernel<T, DH, kMaxWaves>), dim3(p.nwg), dim3(kMaxWaves * kWave),
                       0, st, p);
    if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    if (p.nsplit > 1) {
        const size_t rows = (size_t)p.B * p.Hq * p.T;
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
    return attn_plan(B, Hq, Hkv, Lcap, dh, T, dtype).total;
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
