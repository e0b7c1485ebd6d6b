// Accepted-path KV commit on gfx950.
//
// After acceptance the sequence grows by the root token and the accepted
// candidates (page "Medusa：基于多Token预测的LLM推理加速", section 3.1, step 4
// of its decode loop: the accepted tokens extend the sequence; aiunderstanding
// page, section ディープダイブ: the longest matching prefix is kept).  The tree
// pass already computed their keys and values, so committing them is a gather:
// the K and V rows of the path root -> best_node[b] (in depth order) go to
// cache positions L_b, L_b + 1, ..., and L_b advances by the path length.
//
// One workgroup per sequence: the parent table (passed by value in the
// kernel arguments) goes to LDS and thread 0 walks the path of best_node[b]
// there; then every thread copies 16-byte pieces of the path rows of all kv
// heads, with kCommitU loads in flight before their stores; thread 0
// finally advances L_b.  Only the sequence's own workgroup reads or writes L_b, and its
// write comes after a barrier that follows every read, so the update in
// place needs no ordering between workgroups.
#include "common.h"

namespace medusa {
namespace {

constexpr int kCommitThreads = 1024;
constexpr int kCommitU = 4;

struct CommitParams {
    char *kc, *vc;
    int32_t *prefix_len;
    const char *kt, *vt;
    const int32_t *best;
    int32_t *committed;
    int B, Hkv, Lcap, T, rowbytes;
    uint8_t parent[MEDUSA_MAX_TREE];   // 255 marks the root (never a parent: parent < n <= 255)
};

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitParams p) {
    __shared__ int path[MEDUSA_MAX_TREE];
    __shared__ uint8_t par[MEDUSA_MAX_TREE];
    __shared__ int s_n;
    const int b = blockIdx.x, tid = threadIdx.x;
    // the parent table, L_b and best_node[b] are loaded together
    if (tid < p.T) par[tid] = p.parent[tid];
    const int L = p.prefix_len[b], best = p.best[b];
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        if (L >= 0 && L <= p.Lcap && best >= 0 && best < p.T) {
            int depth = 0;
            for (int a = best; par[a] != 255 && depth < p.T; a = par[a]) ++depth;
            if (L + depth + 1 <= p.Lcap) {
                n = depth + 1;
                for (int a = best, j = depth; j >= 0; --j) {
                    path[j] = a;
                    if (j > 0) a = par[a];
                }
            }
        }
        s_n = n;
    }
    __syncthreads();
    const int n = s_n;
    const int cpr = p.rowbytes / 16;                  // 16-byte pieces per row
    const int total = 2 * p.Hkv * n * cpr;
    for (int c0 = tid; c0 < total; c0 += kCommitU * kCommitThreads) {
        u32x4 v[kCommitU];
        size_t dst[kCommitU];
#pragma unroll
        for (int u = 0; u < kCommitU; ++u) {
            int c = c0 + u * kCommitThreads;
            c = c < total ? c : total - 1;            // clamped duplicates store the same bytes
            const int q = c % cpr;
            const int j = (c / cpr) % n;
            const int hk = c / (cpr * n);             // kv * Hkv + h
            const int kv = hk / p.Hkv, h = hk % p.Hkv;
            const size_t head = (size_t)b * p.Hkv + h;
            const char *src = (kv ? p.vt : p.kt) + ((head * p.T + path[j]) * p.rowbytes + q * 16);
            v[u] = ld16(src);
            dst[u] = ((head * p.Lcap + L + j) * p.rowbytes + q * 16) | ((size_t)kv << 63);
        }
#pragma unroll
        for (int u = 0; u < kCommitU; ++u) {
            const bool is_v = (dst[u] >> 63) != 0;
            st16((is_v ? p.vc : p.kc) + (dst[u] & ~((size_t)1 << 63)), v[u]);
        }
    }
    __syncthreads();
    if (tid == 0) {
        if (n > 0) p.prefix_len[b] = L + n;
        if (p.committed) p.committed[b] = n;
    }
}

}  // namespace
}  // namespace medusa

using namespace medusa;

extern "C" int tree_commit_kv(void *k_cache, void *v_cache, int32_t *prefix_len,
                              const void *k_tree, const void *v_tree, const int32_t *best_node,
                              const int32_t *parent, int B, int Hkv, int Lcap, int dh, int T,
                              int dtype, int32_t *committed, void *stream) {
    if (!k_cache || !v_cache || !prefix_len || !k_tree || !v_tree || !best_node || !parent)
        return MEDUSA_ERR_NULL;
    if (dtype != MEDUSA_F32 && dtype != MEDUSA_BF16) return MEDUSA_ERR_DTYPE;
    const int es = dtype == MEDUSA_BF16 ? 2 : 4;
    if (B < 1 || Hkv < 1 || Lcap < 0 || dh < 1 || (dh * es) % 16 != 0 || T < 1 ||
        T > MEDUSA_MAX_TREE)
        return MEDUSA_ERR_SHAPE;
    if (parent[0] != -1) return MEDUSA_ERR_TREE;
    for (int n = 1; n < T; ++n)
        if (parent[n] < 0 || parent[n] >= n) return MEDUSA_ERR_TREE;
    CommitParams p;
    p.kc = (char *)k_cache;
    p.vc = (char *)v_cache;
    p.prefix_len = prefix_len;
    p.kt = (const char *)k_tree;
    p.vt = (const char *)v_tree;
    p.best = best_node;
    p.committed = committed;
    p.B = B;
    p.Hkv = Hkv;
    p.Lcap = Lcap;
    p.T = T;
    p.rowbytes = dh * es;
    for (int i = 0; i < MEDUSA_MAX_TREE; ++i)
        p.parent[i] = i < T && parent[i] >= 0 ? (uint8_t)parent[i] : (uint8_t)255;
    hipLaunchKernelGGL(commit_kernel, dim3((unsigned)B), dim3(kCommitThreads), 0,
                       (hipStream_t)stream, p);
    return hipGetLastError() == hipSuccess ? MEDUSA_OK : MEDUSA_ERR_LAUNCH;
}
