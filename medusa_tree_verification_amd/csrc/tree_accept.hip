// Acceptance on gfx950: check every candidate against its parent's logits
// row and keep the longest valid path.
//
//  greedy  (temperature 0): a candidate is valid iff it is the argmax of the
//          parent's row (paper explainer page, end of the typical-acceptance
//          section: argmax comparison, lossless);
//  typical: p = softmax(row / temperature), H = -sum p ln p, valid iff
//          p(x) > min(eps, delta * exp(-H))  (same section, its inequality and
//          the defaults eps = 0.09, delta = 0.6).
// The accepted prefix stops at the first rejected token of a path (Chinese
// tutorial page, section 5.3 verification loop) and the longest such path
// wins (aiunderstanding page: accept the longest matching prefix).
//
// Kernel 1 (stats): one workgroup per (vocabulary chunk, node, sequence);
//   nodes without children exit at once.  A single streaming pass over the
//   chunk of the node's logits row records the raw maximum and its index and
//   the running softmax statistics in the log2 domain, m = max z,
//   S = sum 2^(z-m), A = sum 2^(z-m) (z-m) with z = x log2(e) / temperature,
//   so that H = (log2 S - A/S) ln 2.  It also records the token of each
//   child of the node and, in typical mode, the child token's logit (by the
//   chunk that holds it).  Many small workgroups keep the HBM busy even when
//   a batch has few internal nodes.
// Kernel 2 (finish): one workgroup per sequence loads, in one round, the
//   node tokens, the chunk statistics of the internal nodes and the child
//   logits; merges the statistics per node; decides every child; ANDs the
//   valid bits up each node's path; picks the deepest reachable node (lowest
//   index on ties) and writes the accepted tokens, the node tokens and the
//   next token (the best node's argmax: from its statistics when it has
//   children, else from one pass over its row).
// Depth, sibling rank and the has-children flag of every node come from the
// host, which validates the tree anyway.
#include "common.h"

namespace medusa {
namespace {

constexpr int kThreads = 256;        // stats kernel
constexpr int kFinThreads = 1024;    // finish kernel (4 per node for the merges; wide row scan)
constexpr int kMergeLanes = kFinThreads / MEDUSA_MAX_TREE;
constexpr size_t kLeafStatBytes = 16u << 20;   // leaf rows up to this size go through the stats pass
constexpr int kUnroll = 8;           // 16-byte loads in flight per thread (stats)
constexpr int kScanUnroll = 16;      // 16-byte loads in flight per thread (finish row scan)
constexpr int kChunkAlign = 2048;    // vocabulary chunk granularity (elements)
constexpr int kTargetStatWG = 2048;  // aim for about this many stats workgroups
constexpr int kMaxStats = 2048;      // T * nchunk bound (LDS of the finish kernel)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct RowStat {           // 32 bytes
    float xmax;            // largest raw logit of the chunk
    int arg;               // its index (smallest on ties)
    float m, S, A;         // softmax statistics (typical mode)
    float pad[3];
};

struct AcceptParams {
    const void *logits;
    const int32_t *topk;
    RowStat *stats;        // [B][T][nchunk]
    float *childz;         // [B][T] raw logit of node c's token in its parent's row (typical)
    int32_t *ctok;         // [B][T] token of node c (written by its parent's first chunk)
    int32_t *accept_len, *best_node, *accepted, *node_tokens, *next_token;
    int B, T, V, K, s, mode, nchunk, chunk;
    int leaves;            // 1: the stats pass also covers leaf rows (argmax only)
    float zscale;          // log2(e) / temperature
    float eps, delta;
    uint8_t parent[MEDUSA_MAX_TREE];  // 255 marks the root (never a parent: parent < n <= 255)
    uint8_t rank[MEDUSA_MAX_TREE];    // sibling rank: index into the depth's top-s list
    uint8_t depth[MEDUSA_MAX_TREE];
    uint32_t internal[MEDUSA_MAX_TREE / 32];  // bit n: node n has children
    uint8_t rows[MEDUSA_MAX_TREE];    // the nodes whose rows the stats pass reads
    int nrows;
};

__device__ __forceinline__ bool has_children(const AcceptParams &p, int n) {
    return (p.internal[n >> 5] >> (n & 31)) & 1u;
}

// (value, index) argmax with the smaller index winning ties
struct ArgMax {
    float v;
    int i;
    __device__ void add(float x, int j) {
        if (x > v || (x == v && j < i)) {
            v = x;
            i = j;
        }
    }
};

// running softmax statistics in log2 units
struct SoftStats {
    float m, S, A;
    __device__ void merge(float m2, float S2, float A2) {
        if (S2 == 0.f) return;
        if (S == 0.f) {
            m = m2;
            S = S2;
            A = A2;
            return;
        }
        const float M = fmaxf(m, m2);
        const float d1 = m - M, d2 = m2 - M;
        const float f1 = exp2f(d1), f2 = exp2f(d2);
        A = (A + d1 * S) * f1 + (A2 + d2 * S2) * f2;
        S = S * f1 + S2 * f2;
        m = M;
    }
};

template <int NT>
__device__ __forceinline__ ArgMax block_argmax(ArgMax a, ArgMax *sh) {
    for (int m = 32; m >= 1; m >>= 1) {
        ArgMax o{__shfl_xor(a.v, m), __shfl_xor(a.i, m)};
        a.add(o.v, o.i);
    }
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (lane == 0) sh[wave] = a;
    __syncthreads();
    ArgMax r = sh[0];
    for (int w = 1; w < NT / kWave; ++w) r.add(sh[w].v, sh[w].i);
    __syncthreads();
    return r;
}

// Argmax over 16-byte chunks: the best chunk's maximum and its first element
// index.  The first chunk is always taken; later ones only when strictly
// larger, so on ties the earlier chunk wins.  The element index is resolved
// once per workgroup, after the block reduction has picked the winning chunk
// (resolve_chunk: one thread reads that chunk again), which costs fewer
// operations per chunk than carrying its bits.
struct ChunkArgMax {
    float v;
    int base;      // element index of the chunk's first element; -1: none yet
    __device__ __forceinline__ void add(float cm, int b) {
        const bool take = base < 0 || cm > v;
        v = take ? cm : v;
        base = take ? b : base;
    }
};
// r: the block's winning (chunk maximum, chunk start) of row; the first
// element of that chunk equal to the maximum (within a chunk, the earlier
// element wins ties, as across chunks).
template <typename T>
__device__ __forceinline__ ArgMax resolve_chunk(ArgMax r, const T *__restrict__ row) {
    if (r.i == 0x7FFFFFFF) return r;
    constexpr int E = Elem<T>::kPer16B;
    const u32x4 bits = ld16(row + r.i);
    int e0 = E - 1;
#pragma unroll
    for (int e = E - 1; e >= 0; --e) e0 = chunk_elem<T>(bits, e) == r.v ? e : e0;
    r.i += e0;
    return r;
}

// One 16-byte chunk (E elements from index base): argmax, and (typical) the
// softmax statistics of x * zs with one fused multiply-add per element.
template <typename T>
__device__ __forceinline__ void add_chunk_fast(const u32x4 &c, int base, bool typical, float zs,
                                               ChunkArgMax &cam, SoftStats &st) {
    constexpr int E = Elem<T>::kPer16B;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = chunk_elem<T>(c, e);
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) cm = fmaxf(cm, x[e]);
    cam.add(cm, base);
    if (typical) {
        const float cms = cm * zs;   // zs > 0: the maximum of the scaled chunk
        if (cms > st.m) {
            const float d = st.m - cms;
            if (st.S != 0.f) {
                const float f = fast_exp2(d);
                st.A = (st.A + d * st.S) * f;
                st.S *= f;
            }
            st.m = cms;
        }
        const float nm = -st.m;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float dd = fmaf(x[e], zs, nm);
            const float ex = fast_exp2(dd);
            st.S += ex;
            st.A = fmaf(ex, dd, st.A);
        }
    }
}

// one element of a buffer as fp32 (offsets past the buffer read 0)
template <typename T>
__device__ __forceinline__ float buf_elem(__amdgpu_buffer_rsrc_t r, uint32_t i);
template <>
__device__ __forceinline__ float buf_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t i) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, i * 4u, 0, 0));
}
template <>
__device__ __forceinline__ float buf_elem<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t i) {
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, i * 2u, 0, 0));
}

// Raw argmax and (typical) softmax statistics of row[lo, hi), this thread's
// share of the whole workgroup's pass.  Returns true when am is chunk-level
// (index: the chunk's first element; resolve_chunk after the block
// reduction), false when it is element-level.  Loads go through a buffer resource
// over exactly [lo, hi), so they need no predicate (past the end they read 0)
// and all U of them are in flight together; only the accumulation is
// predicated.  16-byte loads need V % E == 0 (rows then start 16-byte
// aligned) and E-aligned bounds; otherwise element loads.
template <typename T, int U = kUnroll, int NT = kThreads>
__device__ __forceinline__ bool row_stats(const T *__restrict__ row, int lo, int hi, int V,
                                          bool typical, float zs, ArgMax &am, SoftStats &st) {
    constexpr int E = Elem<T>::kPer16B;
    const auto rs = make_rsrc(row + lo, (uint32_t)(hi - lo) * (uint32_t)sizeof(T));
    if ((V % E) == 0 && (lo % E) == 0 && (hi % E) == 0) {
        const int nch = (hi - lo) / E;
        ChunkArgMax cam{-INFINITY, -1};
        for (int base = (int)threadIdx.x; base < nch; base += U * NT) {
            u32x4 c[U];
#pragma unroll
            for (int u = 0; u < U; ++u) c[u] = buf_ld16(rs, (uint32_t)(base + u * NT) * 16u);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ch = base + u * NT;
                if (ch < nch) add_chunk_fast<T>(c[u], lo + ch * E, typical, zs, cam, st);
            }
        }
        if (cam.base >= 0) am = ArgMax{cam.v, cam.base};
        return true;
    }
    {
        const int n = hi - lo;
        for (int base = (int)threadIdx.x; base < n; base += U * NT) {
            float x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = buf_elem<T>(rs, (uint32_t)(base + u * NT));
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = base + u * NT;
                if (v < n) {
                    am.add(x[u], lo + v);
                    if (typical) st.merge(x[u] * zs, 1.f, 0.f);
                }
            }
        }
    }
    return false;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void accept_stats_kernel(AcceptParams p) {
    __shared__ ArgMax red[kThreads / kWave];
    __shared__ float redS[3][kThreads / kWave];
    static_assert(kThreads >= MEDUSA_MAX_TREE && kFinThreads % MEDUSA_MAX_TREE == 0, "one thread per tree node");
    const int j = blockIdx.x, n = p.rows[blockIdx.y], b = blockIdx.z;
    const bool internal = has_children(p, n);

    const int lo = j * p.chunk;
    const int hi = lo + p.chunk < p.V ? lo + p.chunk : p.V;
    const bool typical = p.mode != MEDUSA_GREEDY;
    const T *row = (const T *)p.logits + ((size_t)b * p.T + n) * p.V;
    // thread c looks up node c's token (loads issued unconditionally, before
    // the row pass, so that their latency hides under it)
    const int c = threadIdx.x < p.T ? (int)threadIdx.x : 0;
    const int cpar = p.parent[c], cdep = p.depth[c];
    const int tok = p.topk[((size_t)b * p.K + (cdep > 0 ? cdep - 1 : 0)) * p.s + p.rank[c]];
    ArgMax am{-INFINITY, 0x7FFFFFFF};
    SoftStats st{-INFINITY, 0.f, 0.f};
    const bool st_needed = typical && internal;   // softmax statistics: internal rows only
    const bool chunked = row_stats<T>(row, lo, hi, p.V, st_needed, p.zscale, am, st);
    if ((int)threadIdx.x < p.T && c > 0 && cpar == n) {
        // the tokens of n's children, and (typical) each one's logit in this row
        if (j == 0) p.ctok[(size_t)b * p.T + c] = tok;
        if (typical && tok >= lo && tok < hi) p.childz[(size_t)b * p.T + c] = Elem<T>::to_f32(row[tok]);
    }

    ArgMax r = block_argmax<kThreads>(am, red);
    if (chunked && threadIdx.x == 0) r = resolve_chunk<T>(r, row);
    if (st_needed) {
        for (int m = 32; m >= 1; m >>= 1) {
            const float m2 = __shfl_xor(st.m, m), S2 = __shfl_xor(st.S, m), A2 = __shfl_xor(st.A, m);
            st.merge(m2, S2, A2);
        }
        const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
        if (lane == 0) {
            redS[0][wave] = st.m;
            redS[1][wave] = st.S;
            redS[2][wave] = st.A;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            SoftStats tot{redS[0][0], redS[1][0], redS[2][0]};
            for (int w = 1; w < kThreads / kWave; ++w) tot.merge(redS[0][w], redS[1][w], redS[2][w]);
            st = tot;
        }
    }
    if (threadIdx.x == 0) {
        RowStat out;
        out.xmax = r.v;
        out.arg = r.i;
        out.m = st.m;
        out.S = st.S;
        out.A = st.A;
        out.pad[0] = out.pad[1] = out.pad[2] = 0.f;
        p.stats[((size_t)b * p.T + n) * p.nchunk + j] = out;
    }
}

template <typename T>
__global__ __launch_bounds__(kFinThreads) void accept_finish_kernel(AcceptParams p) {
    __shared__ uint8_t par[MEDUSA_MAX_TREE], dep[MEDUSA_MAX_TREE], valid[MEDUSA_MAX_TREE];
    __shared__ uint8_t isint[MEDUSA_MAX_TREE];
    __shared__ int ntok[MEDUSA_MAX_TREE];     // token of every node (root: -1)
    __shared__ float cz[MEDUSA_MAX_TREE];     // its logit in the parent's row (typical)
    __shared__ RowStat sst[kMaxStats];        // this sequence's chunk statistics
    __shared__ int marg[MEDUSA_MAX_TREE];     // merged, per internal node
    __shared__ float mm[MEDUSA_MAX_TREE], mS[MEDUSA_MAX_TREE], mthr[MEDUSA_MAX_TREE];
    __shared__ float lp[MEDUSA_MAX_TREE];     // ln p of every node's token (log-likelihood mode)
    __shared__ unsigned long long keys[kFinThreads / kWave];
    __shared__ ArgMax red[kFinThreads / kWave];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const bool typical = p.mode != MEDUSA_GREEDY;

    // global loads, issued before any wait: the per-node tables, tokens and
    // child logits, then the chunk statistics (every record of the sequence;
    // leaves' records are never read)
    // (loaded into registers here, written to LDS after the record loads
    // are out)
    int rpar = 255, rint = 0, rdep = 0, rtok = -1;
    float rcz = 0.f;
    if (tid < p.T) {
        rpar = p.parent[tid];
        rint = has_children(p, tid);
        rdep = p.depth[tid];
        // node tokens and child logits from the statistics pass (the root has
        // neither; with T == 1 there was no statistics pass)
        if (tid > 0) {
            rtok = p.ctok[(size_t)b * p.T + tid];
            rcz = p.childz[(size_t)b * p.T + tid];
        }
    }
    {
        constexpr int kStageU = 2;   // record loads in flight per thread
        const int nrec = p.T * p.nchunk;
        const RowStat *src = p.stats + (size_t)b * nrec;
        for (int i0 = tid; i0 < nrec; i0 += kStageU * kFinThreads) {
            // indices past the end are clamped to the last record, whose
            // copy is then written again with the same value: no predicate,
            // so that every load is issued before the first wait
            RowStat r[kStageU];
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = i0 + u * kFinThreads;
                r[u] = src[i < nrec ? i : nrec - 1];
            }
#pragma unroll
            for (int u = 0; u < kStageU; ++u) {
                const int i = i0 + u * kFinThreads;
                sst[i < nrec ? i : nrec - 1] = r[u];
            }
        }
    }
    if (tid < p.T) {
        par[tid] = (uint8_t)rpar;
        isint[tid] = (uint8_t)rint;
        dep[tid] = (uint8_t)rdep;
        ntok[tid] = rtok;
        cz[tid] = rcz;
    }
    __syncthreads();
    // merged statistics of each node that has records (internal nodes; all
    // nodes when the stats pass covered the leaves), and each internal
    // node's acceptance threshold: kMergeLanes adjacent lanes per node, each
    // merging every kMergeLanes-th chunk, then combined by shuffles
    {
        const int n = tid / kMergeLanes, q = tid % kMergeLanes;
        const bool has = n < p.T && (isint[n] || p.leaves);
        ArgMax am{-INFINITY, 0x7FFFFFFF};
        SoftStats st{-INFINITY, 0.f, 0.f};
        if (has) {
            for (int j = q; j < p.nchunk; j += kMergeLanes) {
                const RowStat &r = sst[n * p.nchunk + j];
                am.add(r.xmax, r.arg);
                if (typical && isint[n]) st.merge(r.m, r.S, r.A);
            }
        }
#pragma unroll
        for (int m = 1; m < kMergeLanes; m <<= 1) {
            const ArgMax o{__shfl_xor(am.v, m), __shfl_xor(am.i, m)};
            am.add(o.v, o.i);
            const float m2 = __shfl_xor(st.m, m), S2 = __shfl_xor(st.S, m), A2 = __shfl_xor(st.A, m);
            st.merge(m2, S2, A2);
        }
        if (has && q == 0) {
            marg[n] = am.i;
            if (typical && isint[n]) {
                const float H = (log2f(st.S) - st.A / st.S) * kLn2;   // nats
                mm[n] = st.m;
                mS[n] = st.S;
                mthr[n] = fminf(p.eps, p.delta * expf(-H));
            }
        }
    }
    __syncthreads();
    // valid bit of every node (the root counts as valid)
    if (tid < p.T) {
        const int c = tid;
        bool ok = true;
        if (c > 0) {
            const int pn = par[c];
            const int tok = ntok[c];
            float l = -INFINITY;
            if (!typical) {
                ok = tok == marg[pn];
            } else if (tok >= 0 && tok < p.V) {
                const float d = cz[c] * p.zscale - mm[pn];   // log2 units
                ok = exp2f(d) / mS[pn] > mthr[pn];
                l = d * kLn2 - logf(mS[pn]);                 // ln p(tok)
            } else {
                ok = false;
            }
            lp[c] = l;
        } else {
            lp[c] = 0.f;
        }
        valid[c] = ok;
    }
    __syncthreads();

    // deepest node whose path is all valid; equal depths: the larger path
    // log-likelihood in log-likelihood mode, then the lower index.  Key:
    // depth (bits 56..63) | order-preserving bits of the score (24..55) |
    // 0xFFFF - node (0..15); 0 marks "not valid" (every valid key is > 0).
    unsigned long long key = 0ull;
    if (tid < p.T) {
        const int n = tid;
        bool ok = true;
        float sc = 0.f;
        for (int a = n, g = 0; a != 0 && g <= p.T; a = par[a], ++g) {
            ok = ok && valid[a] != 0;
            sc += lp[a];
        }
        if (ok) {
            uint32_t ord = 0u;
            if (p.mode == MEDUSA_TYPICAL_LOGLIK) {
                const uint32_t u = __float_as_uint(sc);
                ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // monotone in sc
            }
            key = ((unsigned long long)dep[n] << 56) | ((unsigned long long)ord << 24) |
                  (unsigned long long)(0xFFFF - n);
        }
        if (p.node_tokens) p.node_tokens[(size_t)b * p.T + n] = ntok[n];
    }
    for (int m = 32; m >= 1; m >>= 1) {
        const unsigned long long o = __shfl_xor(key, m);
        key = o > key ? o : key;
    }
    const int lane = tid % kWave, wave = tid / kWave;
    if (lane == 0) keys[wave] = key;
    __syncthreads();
    unsigned long long best_key = keys[0];
    for (int w = 1; w < kFinThreads / kWave; ++w) best_key = keys[w] > best_key ? keys[w] : best_key;
    const int best = 0xFFFF - (int)(best_key & 0xFFFFull);
    const int bdep = dep[best];
    if (tid == 0) {
        p.accept_len[b] = bdep;
        p.best_node[b] = best;
    }
    if (tid < p.K) {
        int tok = -1;
        if (tid < bdep) {
            int a = best;
            for (int g = 0; dep[a] > tid + 1 && g <= p.T; ++g) a = par[a];
            tok = ntok[a];
        }
        p.accepted[(size_t)b * p.K + tid] = tok;
    }
    if (!p.next_token) return;
    if (isint[best] || p.leaves) {
        if (tid == 0) p.next_token[b] = marg[best];
        return;
    }
    const T *row = (const T *)p.logits + ((size_t)b * p.T + best) * p.V;
    ArgMax am{-INFINITY, 0x7FFFFFFF};
    SoftStats unused{-INFINITY, 0.f, 0.f};
    const bool chunked = row_stats<T, kScanUnroll, kFinThreads>(row, 0, p.V, p.V, false, 0.f, am, unused);
    const ArgMax r = block_argmax<kFinThreads>(am, red);
    if (tid == 0) p.next_token[b] = chunked ? resolve_chunk<T>(r, row).i : r.i;
}

// ---------------------------------------------------------------- bonus token
// The bonus token drawn from p = softmax(logits[b][rows[b]] / temperature)
// (page "Medusa：基于多Token预测的LLM推理加速", section 3.3: sampled
// verification draws from the tempered softmax) by inversion with the
// caller's uniform u[b]: the first token whose cumulative probability
// exceeds u.  One workgroup per sequence: pass 1 finds the row maximum m
// of z = x log2(e) / temperature; pass 2 has every wave sum 2^(z - m) over
// its own contiguous sixteenth of the row; the wave whose range holds the
// target u * S rescans it in groups of 64 with an inclusive lane scan.
// All sums run in a fixed order, so the draw is reproducible.
constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kSampleU = 8;

struct SampleParams {
    const void *logits;
    const int32_t *rows;
    const float *u;
    int32_t *token;
    int B, T, V;
    float zscale;    // log2(e) / temperature
};

template <typename T>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(SampleParams p) {
    __shared__ float red[kSampleWaves];
    __shared__ float wsum[kSampleWaves];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int r = p.rows[b];
    const float u = p.u[b];
    if (r < 0 || r >= p.T || !(u >= 0.f && u < 1.f)) {
        if (tid == 0) p.token[b] = -1;
        return;
    }
    const T *row = (const T *)p.logits + ((size_t)b * p.T + r) * p.V;
    const auto rs = make_rsrc(row, (uint32_t)p.V * (uint32_t)sizeof(T));
    const float zs = p.zscale;

    // pass 1: row maximum (in z units)
    float mx = -INFINITY;
    for (int v0 = tid; v0 < p.V; v0 += kSampleU * kSampleThreads) {
        float x[kSampleU];
#pragma unroll
        for (int k = 0; k < kSampleU; ++k) x[k] = buf_elem<T>(rs, (uint32_t)(v0 + k * kSampleThreads));
#pragma unroll
        for (int k = 0; k < kSampleU; ++k)
            if (v0 + k * kSampleThreads < p.V) mx = fmaxf(mx, x[k] * zs);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float m = red[0];
    for (int w = 1; w < kSampleWaves; ++w) m = fmaxf(m, red[w]);

    // pass 2: each wave's share of S = sum 2^(z - m)
    const int per = (p.V + kSampleWaves - 1) / kSampleWaves;
    const int lo = wave * per < p.V ? wave * per : p.V;
    const int hi = lo + per < p.V ? lo + per : p.V;
    float sum = 0.f;
    for (int v0 = lo + lane; v0 < hi; v0 += kSampleU * kWave) {
        float x[kSampleU];
#pragma unroll
        for (int k = 0; k < kSampleU; ++k) x[k] = buf_elem<T>(rs, (uint32_t)(v0 + k * kWave));
#pragma unroll
        for (int k = 0; k < kSampleU; ++k)
            if (v0 + k * kWave < hi) sum += fast_exp2(x[k] * zs - m);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
    if (lane == 0) wsum[wave] = sum;
    __syncthreads();

    // the wave whose range holds the target (every thread finds the same one)
    float S = 0.f;
    for (int w = 0; w < kSampleWaves; ++w) S += wsum[w];
    const float target = u * S;
    int wsel = -1, wlast = 0;
    float cum = 0.f, cum_last = 0.f;
    for (int w = 0; w < kSampleWaves; ++w) {
        if (wsum[w] > 0.f) {
            wlast = w;
            cum_last = cum;
            if (wsel < 0 && cum + wsum[w] > target) {
                wsel = w;
                break;
            }
        }
        cum += wsum[w];
    }
    if (wsel < 0) {   // rounding put the target past the last share: take that share
        wsel = wlast;
        cum = cum_last;
    }
    if (wave != wsel) return;

    // rescan the share in groups of 64 with an inclusive lane scan
    int tok = hi - 1;
    float run = cum;
    for (int base = lo; base < hi; base += kWave) {
        const int v = base + lane;
        const float x = buf_elem<T>(rs, (uint32_t)v);
        float incl = v < hi ? fast_exp2(x * zs - m) : 0.f;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const float o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        const float total = __shfl(incl, kWave - 1);
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(v < hi && run + incl > target);
        if (hit != 0ull) {
            tok = base + (int)__builtin_ctzll(hit);
            break;
        }
        run += total;
    }
    if (lane == 0) p.token[b] = tok;
}

// host: validate the tree for acceptance (depth <= K, rank < s) and fill in
// every node's depth, sibling rank and has-children flag
int accept_tree(const int32_t *parent, const int32_t *node_rank, int T, int K, int s,
                AcceptParams &p) {
    if (!parent) return MEDUSA_ERR_NULL;
    if (T < 1 || T > MEDUSA_MAX_TREE) return MEDUSA_ERR_SHAPE;
    if (parent[0] != -1) return MEDUSA_ERR_TREE;
    int depth[MEDUSA_MAX_TREE];
    int nchild[MEDUSA_MAX_TREE] = {0};
    for (int i = 0; i < MEDUSA_MAX_TREE; ++i) {
        p.parent[i] = 255;
        p.rank[i] = p.depth[i] = 0;
    }
    for (int i = 0; i < MEDUSA_MAX_TREE / 32; ++i) p.internal[i] = 0u;
    depth[0] = 0;
    for (int n = 1; n < T; ++n) {
        if (parent[n] < 0 || parent[n] >= n) return MEDUSA_ERR_TREE;
        depth[n] = depth[parent[n]] + 1;
        if (depth[n] > K) return MEDUSA_ERR_TREE;
        const int r = node_rank ? node_rank[n] : nchild[parent[n]];
        if (r < 0 || r >= s) return MEDUSA_ERR_TREE;
        nchild[parent[n]]++;
        p.parent[n] = (uint8_t)parent[n];
        p.rank[n] = (uint8_t)r;
        p.depth[n] = (uint8_t)depth[n];
        p.internal[parent[n] >> 5] |= 1u << (parent[n] & 31);
    }
    if (node_rank) {
        for (int n = 1; n < T; ++n)
            for (int m = 1; m < n; ++m)
                if (parent[m] == parent[n] && node_rank[m] == node_rank[n]) return MEDUSA_ERR_TREE;
    }
    return MEDUSA_OK;
}

// Vocabulary chunks per row: enough stats workgroups to fill the GPU (about
// half the nodes of a tree have children), chunks of whole kChunkAlign
// elements, at most kMaxStats records per sequence.  Depends on (B, T, V)
// only, so the workspace size does too.
void accept_chunks(int B, int T, int V, int *nchunk, int *chunk) {
    const long long rows = (long long)B * (T > 1 ? (T + 1) / 2 : 1);
    int want = (int)((kTargetStatWG + rows - 1) / rows);
    const int vmax = (V + kChunkAlign - 1) / kChunkAlign;
    const int lmax = kMaxStats / T;
    if (want > vmax) want = vmax;
    if (want > lmax) want = lmax;
    if (want < 1) want = 1;
    int ch = (V + want - 1) / want;
    ch = (ch + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
    *chunk = ch;
    *nchunk = (V + ch - 1) / ch;
}

}  // namespace
}  // namespace medusa

using namespace medusa;

// workspace: chunk statistics [B][T][nchunk], child logits [B][T], child tokens [B][T]
static size_t accept_stats_bytes(int B, int T, int V) {
    int nchunk, chunk;
    accept_chunks(B, T, V, &nchunk, &chunk);
    return align_up((size_t)B * T * nchunk * sizeof(RowStat), 256);
}

extern "C" size_t tree_accept_workspace_bytes(int B, int T, int V, int K, int s) {
    if (B < 1 || T < 1 || T > MEDUSA_MAX_TREE || V < 1 || K < 0 || s < 1) return 0;
    return accept_stats_bytes(B, T, V) + 2 * align_up((size_t)B * T * sizeof(float), 256);
}

extern "C" int tree_accept(const void *logits, const int32_t *topk_ids, const int32_t *parent,
                           const int32_t *node_rank, int B, int T, int V, int K, int s, int dtype,
                           int mode, float temperature, float eps, float delta,
                           int32_t *accept_len, int32_t *best_node, int32_t *accepted_tokens,
                           int32_t *node_tokens, int32_t *next_token, void *ws, size_t ws_bytes,
                           void *stream) {
    if (!logits || !topk_ids || !accept_len || !best_node || !accepted_tokens)
        return MEDUSA_ERR_NULL;
    if (dtype != MEDUSA_F32 && dtype != MEDUSA_BF16) return MEDUSA_ERR_DTYPE;
    if (B < 1 || V < 1 || K < 0 || K > MEDUSA_MAX_HEADS || s < 1 || s > 255)
        return MEDUSA_ERR_SHAPE;
    if (mode != MEDUSA_GREEDY && mode != MEDUSA_TYPICAL && mode != MEDUSA_TYPICAL_LOGLIK)
        return MEDUSA_ERR_PARAM;
    if (mode != MEDUSA_GREEDY &&
        !(temperature > 0.f && temperature < INFINITY && eps > 0.f && eps < INFINITY &&
          delta > 0.f && delta < INFINITY))
        return MEDUSA_ERR_PARAM;
    AcceptParams p;
    const int st = accept_tree(parent, node_rank, T, K, s, p);
    if (st != MEDUSA_OK) return st;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < tree_accept_workspace_bytes(B, T, V, K, s))
        return MEDUSA_ERR_WORKSPACE;

    p.logits = logits;
    p.topk = topk_ids;
    p.stats = (RowStat *)ws;
    p.childz = (float *)((char *)ws + accept_stats_bytes(B, T, V));
    p.ctok = (int32_t *)((char *)p.childz + align_up((size_t)B * T * sizeof(float), 256));
    p.accept_len = accept_len;
    p.best_node = best_node;
    p.accepted = accepted_tokens;
    p.node_tokens = node_tokens;
    p.next_token = next_token;
    p.B = B;
    p.T = T;
    p.V = V;
    p.K = K;
    p.s = s;
    p.mode = mode;
    p.zscale = mode != MEDUSA_GREEDY ? kLog2e / temperature : 0.f;
    p.eps = eps;
    p.delta = delta;
    accept_chunks(B, T, V, &p.nchunk, &p.chunk);
    {
        int nleaf = 0;
        for (int n = 0; n < T; ++n) nleaf += !((p.internal[n >> 5] >> (n & 31)) & 1u);
        const size_t leaf_bytes = (size_t)B * nleaf * V * (dtype == MEDUSA_BF16 ? 2 : 4);
        p.leaves = T > 1 && leaf_bytes <= kLeafStatBytes;
        p.nrows = 0;
        for (int n = 0; n < T; ++n)
            if (p.leaves || ((p.internal[n >> 5] >> (n & 31)) & 1u)) p.rows[p.nrows++] = (uint8_t)n;
    }
    hipStream_t sm = (hipStream_t)stream;
    if (T > 1) {
        const dim3 grid((unsigned)p.nchunk, (unsigned)p.nrows, (unsigned)B);
        if (dtype == MEDUSA_BF16)
            hipLaunchKernelGGL(accept_stats_kernel<bf16_t>, grid, dim3(kThreads), 0, sm, p);
        else
            hipLaunchKernelGGL(accept_stats_kernel<float>, grid, dim3(kThreads), 0, sm, p);
        if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    }
    if (dtype == MEDUSA_BF16)
        hipLaunchKernelGGL(accept_finish_kernel<bf16_t>, dim3(B), dim3(kFinThreads), 0, sm, p);
    else
        hipLaunchKernelGGL(accept_finish_kernel<float>, dim3(B), dim3(kFinThreads), 0, sm, p);
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
}

extern "C" int medusa_sample_token(const void *logits, const int32_t *rows, const float *u, int B,
                                   int T, int V, int dtype, float temperature, int32_t *token,
                                   void *stream) {
    if (!logits || !rows || !u || !token) return MEDUSA_ERR_NULL;
    if (dtype != MEDUSA_F32 && dtype != MEDUSA_BF16) return MEDUSA_ERR_DTYPE;
    if (B < 1 || T < 1 || V < 1) return MEDUSA_ERR_SHAPE;
    if (!(temperature > 0.f && temperature < INFINITY)) return MEDUSA_ERR_PARAM;
    SampleParams p;
    p.logits = logits;
    p.rows = rows;
    p.u = u;
    p.token = token;
    p.B = B;
    p.T = T;
    p.V = V;
    p.zscale = kLog2e / temperature;
    hipStream_t sm = (hipStream_t)stream;
    if (dtype == MEDUSA_BF16)
        hipLaunchKernelGGL(sample_kernel<bf16_t>, dim3(B), dim3(kSampleThreads), 0, sm, p);
    else
        hipLaunchKernelGGL(sample_kernel<float>, dim3(B), dim3(kSampleThreads), 0, sm, p);
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
}

extern "C" const char *medusa_status_str(int status) {
    switch (status) {
        case MEDUSA_OK: return "ok";
        case MEDUSA_ERR_NULL: return "a required pointer is NULL";
        case MEDUSA_ERR_SHAPE: return "a size is outside the supported range";
        case MEDUSA_ERR_DTYPE: return "unknown dtype";
        case MEDUSA_ERR_TREE: return "parent/node_rank does not describe a valid candidate tree";
        case MEDUSA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MEDUSA_ERR_PARAM: return "bad scalar parameter";
        case MEDUSA_ERR_LAUNCH: return "kernel launch failed";
        case MEDUSA_ERR_SCRATCH:
            return "the problem needs more scratch than the no-allocation entry point holds";
        default: return "unknown status";
    }
}

extern "C" int medusa_abi_version(void) { return 1; }
