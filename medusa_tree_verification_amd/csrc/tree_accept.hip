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
// Kernel 1 (rows): one workgroup per (internal node, sequence).  A single
//   streaming pass over the node's V logits computes the argmax, or the
//   running (max m, S = sum e^(z-m), A = sum e^(z-m)(z-m)) from which
//   H = ln S - A/S, and writes the valid bit of each child.
// Kernel 2 (scan): one workgroup per sequence: each thread takes one node,
//   ANDs the valid bits up its path, a block reduction picks the deepest
//   reachable node (lowest index on ties); then the accepted tokens, the
//   node tokens and the argmax of the best node's row (next token).
#include "common.h"

namespace medusa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;    // 16-byte loads in flight per thread in row scans
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AcceptParams {
    const void *logits;
    const int32_t *topk;
    uint8_t *valid;   // [B][T]
    int32_t *accept_len, *best_node, *accepted, *node_tokens, *next_token;
    int B, T, V, K, s, mode, has_rank;
    float zscale;     // log2(e) / temperature
    float eps, delta;
    uint8_t parent[MEDUSA_MAX_TREE];  // 255 = root
    uint8_t rank[MEDUSA_MAX_TREE];
};

__device__ __forceinline__ void load_tree(const AcceptParams &p, uint8_t *par, uint8_t *dep,
                                          uint8_t *rk) {
    for (int i = threadIdx.x; i < p.T; i += blockDim.x) par[i] = p.parent[i];
    __syncthreads();
    for (int n = threadIdx.x; n < p.T; n += blockDim.x) {
        int d = 0;
        for (int a = n; par[a] != 255 && d <= p.T; a = par[a]) ++d;
        dep[n] = (uint8_t)d;
        int r = 0;
        if (p.has_rank) {
            r = p.rank[n];
        } else if (n > 0) {
            for (int m = 1; m < n; ++m) r += par[m] == par[n];
        }
        rk[n] = (uint8_t)r;
    }
    __syncthreads();
}

__device__ __forceinline__ int node_token(const AcceptParams &p, int b, int n, const uint8_t *dep,
                                          const uint8_t *rk) {
    if (n == 0) return -1;
    return p.topk[((size_t)b * p.K + dep[n] - 1) * p.s + rk[n]];
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

__device__ __forceinline__ ArgMax block_argmax(ArgMax a, ArgMax *sh) {
    for (int m = 32; m >= 1; m >>= 1) {
        ArgMax o{__shfl_xor(a.v, m), __shfl_xor(a.i, m)};
        a.add(o.v, o.i);
    }
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (lane == 0) sh[wave] = a;
    __syncthreads();
    ArgMax r = sh[0];
    for (int w = 1; w < (int)(blockDim.x / kWave); ++w) r.add(sh[w].v, sh[w].i);
    __syncthreads();
    return r;
}

// running softmax statistics in log2 units: m, S = sum 2^(x-m), A = sum 2^(x-m)(x-m)
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

template <typename T>
__device__ __forceinline__ void scan_row_chunk(const u32x4 &c, int base, int mode, float zs,
                                               ArgMax &am, SoftStats &st) {
    constexpr int E = Elem<T>::kPer16B;
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = chunk_elem<T>(c, e);
    if (mode == MEDUSA_GREEDY) {
#pragma unroll
        for (int e = 0; e < E; ++e) am.add(x[e], base + e);
    } else {
        float cm = -INFINITY;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            x[e] *= zs;
            cm = fmaxf(cm, x[e]);
        }
        if (cm > st.m) {
            const float d = st.m - cm;
            if (st.S != 0.f) {
                const float f = fast_exp2(d);
                st.A = (st.A + d * st.S) * f;
                st.S *= f;
            }
            st.m = cm;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float dd = x[e] - st.m;
            const float ex = fast_exp2(dd);
            st.S += ex;
            st.A += ex * dd;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void accept_rows_kernel(AcceptParams p) {
    __shared__ uint8_t par[MEDUSA_MAX_TREE];
    __shared__ int node_sh, node_depth;
    __shared__ uint8_t is_int[kThreads];
    __shared__ int wcount[kThreads / kWave];
    __shared__ int ccount[kThreads / kWave];
    __shared__ int child_tok[MEDUSA_MAX_TREE];   // token of child node c (by index)
    __shared__ ArgMax red[kThreads / kWave];
    __shared__ float redS[3][kThreads / kWave];
    static_assert(kThreads >= MEDUSA_MAX_TREE, "one thread per tree node");
    for (int i = threadIdx.x; i < p.T; i += kThreads) par[i] = p.parent[i];
    const int b = blockIdx.y;

    // this workgroup's node: the blockIdx.x-th node (in index order) that has
    // a child.  Mark parents, then rank the marks with a ballot prefix count.
    if (threadIdx.x == 0) node_sh = -1;
    is_int[threadIdx.x] = 0;
    __syncthreads();
    if (threadIdx.x >= 1 && (int)threadIdx.x < p.T) is_int[par[threadIdx.x]] = 1;
    __syncthreads();
    {
        const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
        const bool mine = is_int[threadIdx.x] != 0;
        const uint64_t bal = __ballot(mine);
        if (lane == 0) wcount[wave] = __popcll(bal);
        __syncthreads();
        int before = __popcll(bal & ((1ull << lane) - 1ull));
        for (int w = 0; w < wave; ++w) before += wcount[w];
        if (mine && before == (int)blockIdx.x) node_sh = threadIdx.x;
    }
    __syncthreads();
    const int n = node_sh;
    if (n < 0) return;
    // the children of n, their ranks (ballot prefix count over child flags, or
    // node_rank) and their tokens: candidate rank(c) of head depth(n)
    if (threadIdx.x == 0) {
        int dn = 0;
        for (int a = n; par[a] != 255 && dn <= p.T; a = par[a]) ++dn;
        node_depth = dn;
    }
    {
        const int c = threadIdx.x;
        const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
        const bool child = c < p.T && c > n && par[c] == n;
        const uint64_t bal = __ballot(child);
        if (lane == 0) ccount[wave] = __popcll(bal);
        __syncthreads();
        if (child) {
            int rank = __popcll(bal & ((1ull << lane) - 1ull));
            for (int w = 0; w < wave; ++w) rank += ccount[w];
            if (p.has_rank) rank = p.rank[c];
            child_tok[c] = p.topk[((size_t)b * p.K + node_depth) * p.s + rank];
        }
        __syncthreads();
    }

    const T *row = (const T *)p.logits + ((size_t)b * p.T + n) * p.V;
    ArgMax am{-INFINITY, 0x7FFFFFFF};
    SoftStats st{-INFINITY, 0.f, 0.f};
    constexpr int E = Elem<T>::kPer16B;
    const bool vec = (p.V % E) == 0;
    if (vec) {
        // whole batches of kUnroll loads per thread, the last one predicated
        const int nch = p.V / E;
        for (int base = threadIdx.x; base < nch; base += kUnroll * kThreads) {
            u32x4 c[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int ch = base + u * kThreads;
                c[u] = ch < nch ? ld16(row + (size_t)ch * E) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int ch = base + u * kThreads;
                if (ch < nch) scan_row_chunk<T>(c[u], ch * E, p.mode, p.zscale, am, st);
            }
        }
    } else {
        for (int v = threadIdx.x; v < p.V; v += kThreads) {
            const float x = Elem<T>::to_f32(row[v]);
            if (p.mode == MEDUSA_GREEDY) {
                am.add(x, v);
            } else {
                st.merge(x * p.zscale, 1.f, 0.f);
            }
        }
    }

    if (p.mode == MEDUSA_GREEDY) {
        const ArgMax r = block_argmax(am, red);
        for (int c = n + 1 + (int)threadIdx.x; c < p.T; c += kThreads)
            if (par[c] == n) p.valid[(size_t)b * p.T + c] = child_tok[c] == r.i;
    } else {
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
        SoftStats tot{redS[0][0], redS[1][0], redS[2][0]};
        for (int w = 1; w < kThreads / kWave; ++w) tot.merge(redS[0][w], redS[1][w], redS[2][w]);
        // H in nats: ln S - (A/S) ln 2  (A in log2 units)
        const float H = (log2f(tot.S) - tot.A / tot.S) * kLn2;
        const float thr = fminf(p.eps, p.delta * expf(-H));
        for (int c = n + 1 + (int)threadIdx.x; c < p.T; c += kThreads) {
            if (par[c] != n) continue;
            const int tok = child_tok[c];
            bool ok = false;
            if (tok >= 0 && tok < p.V) {
                const float z = Elem<T>::to_f32(row[tok]) * p.zscale;
                const float pc = exp2f(z - tot.m) / tot.S;
                ok = pc > thr;
            }
            p.valid[(size_t)b * p.T + c] = ok;
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void accept_scan_kernel(AcceptParams p) {
    __shared__ uint8_t par[MEDUSA_MAX_TREE], dep[MEDUSA_MAX_TREE], rk[MEDUSA_MAX_TREE];
    __shared__ uint8_t valid[MEDUSA_MAX_TREE];
    __shared__ int cand[MEDUSA_MAX_HEADS * 256];
    __shared__ int keys[kThreads / kWave];
    __shared__ ArgMax red[kThreads / kWave];
    const int b = blockIdx.x;
    // this sequence's valid bits and candidate ids, read once into LDS
    for (int n = threadIdx.x; n < p.T; n += kThreads) valid[n] = p.valid[(size_t)b * p.T + n];
    for (int i = threadIdx.x; i < p.K * p.s; i += kThreads) cand[i] = p.topk[(size_t)b * p.K * p.s + i];
    load_tree(p, par, dep, rk);   // ends with a barrier

    int key = -1;  // (depth << 16) | (0xFFFF - node): max = deepest, lowest index
    for (int n = threadIdx.x; n < p.T; n += kThreads) {
        bool ok = true;
        for (int a = n, g = 0; a != 0 && g <= p.T; a = par[a], ++g) ok = ok && valid[a] != 0;
        if (ok) {
            const int k = ((int)dep[n] << 16) | (0xFFFF - n);
            key = k > key ? k : key;
        }
        if (p.node_tokens)
            p.node_tokens[(size_t)b * p.T + n] = n == 0 ? -1 : cand[(dep[n] - 1) * p.s + rk[n]];
    }
    for (int m = 32; m >= 1; m >>= 1) {
        const int o = __shfl_xor(key, m);
        key = o > key ? o : key;
    }
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (lane == 0) keys[wave] = key;
    __syncthreads();
    int best_key = keys[0];
    for (int w = 1; w < kThreads / kWave; ++w) best_key = keys[w] > best_key ? keys[w] : best_key;
    const int best = 0xFFFF - (best_key & 0xFFFF);
    const int bdep = dep[best];
    if (threadIdx.x == 0) {
        p.accept_len[b] = bdep;
        p.best_node[b] = best;
    }
    for (int k = threadIdx.x; k < p.K; k += kThreads) {
        int tok = -1;
        if (k < bdep) {
            int a = best;
            for (int g = 0; dep[a] > k + 1 && g <= p.T; ++g) a = par[a];
            tok = cand[(dep[a] - 1) * p.s + rk[a]];
        }
        p.accepted[(size_t)b * p.K + k] = tok;
    }
    if (!p.next_token) return;
    const T *row = (const T *)p.logits + ((size_t)b * p.T + best) * p.V;
    ArgMax am{-INFINITY, 0x7FFFFFFF};
    constexpr int E = Elem<T>::kPer16B;
    if (p.V % E == 0) {
        const int nch = p.V / E;
        for (int base = threadIdx.x; base < nch; base += kUnroll * kThreads) {
            u32x4 c[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int ch = base + u * kThreads;
                c[u] = ch < nch ? ld16(row + (size_t)ch * E) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int ch = base + u * kThreads;
                if (ch < nch) {
#pragma unroll
                    for (int e = 0; e < E; ++e) am.add(chunk_elem<T>(c[u], e), ch * E + e);
                }
            }
        }
    } else {
        for (int v = threadIdx.x; v < p.V; v += kThreads) am.add(Elem<T>::to_f32(row[v]), v);
    }
    const ArgMax r = block_argmax(am, red);
    if (threadIdx.x == 0) p.next_token[b] = r.i;
}

// host: validate the tree for acceptance (depth <= K, rank < s)
int check_accept_tree(const int32_t *parent, const int32_t *node_rank, int T, int K, int s,
                      int *n_internal) {
    if (!parent) return MEDUSA_ERR_NULL;
    if (T < 1 || T > MEDUSA_MAX_TREE) return MEDUSA_ERR_SHAPE;
    if (parent[0] != -1) return MEDUSA_ERR_TREE;
    int depth[MEDUSA_MAX_TREE];
    int nchild[MEDUSA_MAX_TREE] = {0};
    depth[0] = 0;
    for (int n = 1; n < T; ++n) {
        if (parent[n] < 0 || parent[n] >= n) return MEDUSA_ERR_TREE;
        depth[n] = depth[parent[n]] + 1;
        if (depth[n] > K) return MEDUSA_ERR_TREE;
        const int r = node_rank ? node_rank[n] : nchild[parent[n]];
        if (r < 0 || r >= s) return MEDUSA_ERR_TREE;
        nchild[parent[n]]++;
    }
    if (node_rank) {
        for (int n = 1; n < T; ++n)
            for (int m = 1; m < n; ++m)
                if (parent[m] == parent[n] && node_rank[m] == node_rank[n]) return MEDUSA_ERR_TREE;
    }
    int ni = 0;
    for (int n = 0; n < T; ++n) ni += nchild[n] > 0;
    *n_internal = ni;
    return MEDUSA_OK;
}

}  // namespace
}  // namespace medusa

using namespace medusa;

extern "C" size_t tree_accept_workspace_bytes(int B, int T, int V, int K, int s) {
    if (B < 1 || T < 1 || T > MEDUSA_MAX_TREE || V < 1 || K < 0 || s < 1) return 0;
    (void)K;
    (void)s;
    return align_up((size_t)B * T, 256);
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
    if (mode != MEDUSA_GREEDY && mode != MEDUSA_TYPICAL) return MEDUSA_ERR_PARAM;
    if (mode == MEDUSA_TYPICAL &&
        !(temperature > 0.f && temperature < INFINITY && eps > 0.f && eps < INFINITY &&
          delta > 0.f && delta < INFINITY))
        return MEDUSA_ERR_PARAM;
    int n_internal = 0;
    int st = check_accept_tree(parent, node_rank, T, K, s, &n_internal);
    if (st != MEDUSA_OK) return st;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < tree_accept_workspace_bytes(B, T, V, K, s))
        return MEDUSA_ERR_WORKSPACE;

    AcceptParams p;
    p.logits = logits;
    p.topk = topk_ids;
    p.valid = (uint8_t *)ws;
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
    p.has_rank = node_rank != nullptr;
    p.zscale = mode == MEDUSA_TYPICAL ? kLog2e / temperature : 0.f;
    p.eps = eps;
    p.delta = delta;
    for (int i = 0; i < MEDUSA_MAX_TREE; ++i) {
        p.parent[i] = i < T && parent[i] >= 0 ? (uint8_t)parent[i] : (uint8_t)255;
        p.rank[i] = (node_rank && i < T && i > 0) ? (uint8_t)node_rank[i] : (uint8_t)0;
    }
    hipStream_t sm = (hipStream_t)stream;
    if (n_internal > 0) {
        if (dtype == MEDUSA_BF16)
            hipLaunchKernelGGL(accept_rows_kernel<bf16_t>, dim3(n_internal, B), dim3(kThreads), 0,
                               sm, p);
        else
            hipLaunchKernelGGL(accept_rows_kernel<float>, dim3(n_internal, B), dim3(kThreads), 0,
                               sm, p);
        if (hipGetLastError() != hipSuccess) return MEDUSA_ERR_LAUNCH;
    }
    if (dtype == MEDUSA_BF16)
        hipLaunchKernelGGL(accept_scan_kernel<bf16_t>, dim3(B), dim3(kThreads), 0, sm, p);
    else
        hipLaunchKernelGGL(accept_scan_kernel<float>, dim3(B), dim3(kThreads), 0, sm, p);
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
        default: return "unknown status";
    }
}

extern "C" int medusa_abi_version(void) { return 1; }
