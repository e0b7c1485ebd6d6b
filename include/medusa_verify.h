/*
 * medusa_verify.h -- C ABI of the MI355X (gfx950) Medusa verify step.
 *
 * One Medusa decode step verifies, in a single pass, the candidate tokens
 * proposed by K extra decoding heads on the base model's last hidden state
 * ("Medusa: Simple LLM Inference Acceleration Framework with Multiple
 * Decoding Heads", paper explainer page: head architecture, tree attention,
 * typical acceptance).  The library exports the three compute calls of that
 * step, all asynchronous on a caller-supplied HIP stream:
 *
 *   medusa_heads_topk  K heads H_i(h) = W2_i (SiLU(W1_i h) + h) + top-s
 *   tree_attention     every tree node attends to the KV prefix plus its own
 *                      ancestors (and itself) -- one pass over the tree
 *   tree_accept        greedy or typical acceptance of the longest valid path
 *   medusa_sample_token a sampled bonus token from the best node's row
 *   tree_commit_kv     append the accepted path's K/V rows to the cache
 *   medusa_verify_forward  N attention blocks + LM head over the tree's
 *                      tokens: verification logits from a forward pass
 *
 * Conventions (all calls):
 *  - Every pointer marked "device" is device memory on the current HIP
 *    device; "host" pointers are read during the call only.  The caller owns
 *    all memory; the library never allocates, frees or synchronises.
 *  - Tensors are dense, row-major, with the shapes written next to them.
 *    Weights are [out][in] (torch.nn.Linear layout).  Element type is given
 *    by `dtype`: MEDUSA_F32 (IEEE binary32) or MEDUSA_BF16 (bfloat16, the
 *    upper 16 bits of a binary32).  Index tensors are int32.
 *  - `stream` is a hipStream_t (NULL = the null stream).
 *  - Scratch memory comes from the caller's workspace `ws` of `ws_bytes`
 *    bytes (device, 256-byte aligned), sized by the matching
 *    *_workspace_bytes() call.  Its contents need no initialisation and are
 *    undefined after the call, with one exception: tree_attention leaves
 *    its prefix-length flag in the workspace's first int32 (see there),
 *    which every tree_attention call rewrites and any other call on the
 *    same workspace may overwrite.  Calls that share a workspace must be
 *    ordered on one stream.
 *  - Return value: MEDUSA_OK, or a negative medusa_status.  Argument errors
 *    are detected on the host before anything is enqueued; no output is
 *    touched then.  MEDUSA_ERR_LAUNCH reports a failed kernel launch.
 *  - The library is safe to call from several host threads (on different
 *    workspaces).  Its only global state is the scratch array of
 *    medusa_heads_topk_noalloc (one per GPU) and that array's per-device
 *    address, looked up under a lock on the first such call on a device.
 */
#ifndef MEDUSA_VERIFY_H
#define MEDUSA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;

typedef enum {
    MEDUSA_GREEDY = 0,
    MEDUSA_TYPICAL = 1,
    MEDUSA_TYPICAL_LOGLIK = 2   /* typical; equal-depth paths ranked by log-likelihood */
} medusa_accept_mode;

typedef enum {
    MEDUSA_OK = 0,
    MEDUSA_ERR_NULL = -1,      /* a required pointer is NULL              */
    MEDUSA_ERR_SHAPE = -2,     /* a size is out of the supported range    */
    MEDUSA_ERR_DTYPE = -3,     /* unknown dtype                           */
    MEDUSA_ERR_TREE = -4,      /* parent / node_rank array is not a valid tree */
    MEDUSA_ERR_WORKSPACE = -5, /* workspace missing, misaligned or too small */
    MEDUSA_ERR_PARAM = -6,     /* bad scalar (mode, temperature, eps, delta, scale) */
    MEDUSA_ERR_LAUNCH = -7,    /* a kernel launch failed                  */
    MEDUSA_ERR_SCRATCH = -8    /* needs more than the no-allocation entry point's scratch */
} medusa_status;

/* Supported ranges (checked on the host). */
#define MEDUSA_MAX_BATCH 16     /* heads: B <= 16 (one MFMA column tile) */
#define MEDUSA_MAX_HEADS 16     /* K                                      */
#define MEDUSA_MAX_TOPS 8       /* s                                      */
#define MEDUSA_MAX_TREE 256     /* T, nodes including the root            */
#define MEDUSA_MAX_LAYERS 256   /* N, attention blocks of the forward      */

/* ------------------------------------------------------------------------
 * medusa_heads_topk -- the K Medusa heads and their top-s candidates.
 *
 * Head equation of the paper explainer page (section "Medusa Head
 * architecture"): H_i(h) = W2_i (SiLU(W1_i h) + h), SiLU(x) = x*sigmoid(x),
 * W1_i: d -> d, W2_i: d -> V, no biases (its PyTorch head listing); every
 * head reads the same hidden state h.  Then the s largest logits of every
 * (sequence, head), as candidate tokens for tree depth i+1 (same page,
 * "tree attention": top-s per head, s = 3 recommended).
 *
 *   hidden     device [B][d]        dtype
 *   w1         device [K][d][d]     dtype   ([out][in])
 *   w2         device [K][V][d]     dtype   ([out][in])
 *   logits_out device [B][K][V]     float32, or NULL to skip writing logits
 *   topk_ids   device [B][K][s]     int32: larger logit first, equal logits
 *                                   ordered by smaller token id
 *   topk_vals  device [B][K][s]     float32 logits of topk_ids, or NULL
 *
 * Arithmetic: fp32 accumulation.  In BF16 mode the W2 input
 * z = SiLU(W1 h) + h is rounded once to bf16 (nearest-even); logits are
 * fp32 and not rounded.  Limits: 1 <= B <= 16, 1 <= K <= 16,
 * 128 <= d <= 16384 with d % 128 == 0, s <= V, 1 <= s <= 8.
 * Kernels: stage 1 (W1 stream + SiLU + residual -> z in the workspace),
 * stage 2 (W2 stream on the matrix cores with a fused per-workgroup top-s)
 * and a small merge of each head's per-workgroup lists.
 * ---------------------------------------------------------------------- */
int medusa_heads_topk(const void *hidden, const void *w1, const void *w2, int B, int K, int d,
                      int V, int s, int dtype, float *logits_out, int32_t *topk_ids,
                      float *topk_vals, void *ws, size_t ws_bytes, void *stream);

/* The two stages of medusa_heads_topk as separate calls (same arguments and
 * workspace; stage 2 must follow stage 1 on the same stream and workspace).
 * medusa_heads_topk is exactly stage 1 followed by stage 2. */
int medusa_heads_stage1(const void *hidden, const void *w1, int B, int K, int d, int V, int s,
                        int dtype, void *ws, size_t ws_bytes, void *stream);
int medusa_heads_stage2(const void *w2, int B, int K, int d, int V, int s, int dtype,
                        float *logits_out, int32_t *topk_ids, float *topk_vals, void *ws,
                        size_t ws_bytes, void *stream);

/* The two kernels of medusa_heads_stage2 as separate calls (same arguments
 * and workspace): the W2 stream with a top-s list per (workgroup, head,
 * sequence) left in the workspace, then the merge of those lists into
 * topk_ids / topk_vals.  medusa_heads_stage2 is exactly stream followed by
 * merge on the same stream and workspace; the split lets a caller time the
 * weight stream by itself. */
int medusa_heads_stage2_stream(const void *w2, int B, int K, int d, int V, int s, int dtype,
                               float *logits_out, void *ws, size_t ws_bytes, void *stream);
int medusa_heads_stage2_merge(int B, int K, int d, int V, int s, int dtype, int32_t *topk_ids,
                              float *topk_vals, void *ws, size_t ws_bytes, void *stream);

size_t medusa_heads_topk_workspace_bytes(int B, int K, int d, int V, int s, int dtype);

/* medusa_heads_topk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It allocates nothing: its
 * scratch (z and the per-workgroup top-s lists, the same bytes
 * medusa_heads_topk_workspace_bytes counts) lives in a static device array
 * of medusa_heads_topk_noalloc_max_scratch() bytes (8 MiB) that each GPU the
 * library runs on holds until the process ends.  A problem whose workspace
 * would exceed it is rejected with MEDUSA_ERR_SCRATCH before anything is
 * enqueued (every shape with B <= 16, K <= 8 and d <= 4096 fits).
 * Arguments, limits, results and kernels are those of medusa_heads_topk;
 * the scratch needs no initialisation (every byte read is first written
 * by the same call).  All calls on one GPU share its array: calls that
 * overlap on one GPU (on different streams, or from several host threads
 * without ordering) race and give undefined results; order them on one
 * stream.  The first call on a device looks up the array's device address
 * (MEDUSA_ERR_LAUNCH if that fails). */
int medusa_heads_topk_noalloc(const void *hidden, const void *w1, const void *w2, int B, int K,
                              int d, int V, int s, int dtype, float *logits_out,
                              int32_t *topk_ids, float *topk_vals, void *stream);
size_t medusa_heads_topk_noalloc_max_scratch(void);

/* medusa_heads_topk plus the tree's root token: the base model's own next
 * token, the argmax of its LM head w_lm on the same hidden state (paper
 * explainer page, section "Medusa Headのアーキテクチャ", its diagram: the
 * original LM head gives x_{t+1}, Medusa head i gives x_{t+i+1}).  The LM
 * head's weights ride along in stage 2's weight stream as one more head
 * (input: the hidden state itself, no SiLU block).
 *
 *   w_lm        device [V][d] dtype ([out][in])
 *   root_token  device [B] int32: argmax_v (w_lm h)_v, equal logits ->
 *               smaller id
 *   root_val    device [B] float32 logit of root_token, or NULL
 * Other arguments, limits and the workspace as medusa_heads_topk
 * (logits_out covers the K Medusa heads only). */
int medusa_heads_topk_root(const void *hidden, const void *w1, const void *w2, const void *w_lm,
                           int B, int K, int d, int V, int s, int dtype, float *logits_out,
                           int32_t *topk_ids, float *topk_vals, int32_t *root_token,
                           float *root_val, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * tree_attention -- one attention pass over the candidate tree.
 *
 * Tree-attention section of the paper explainer page: the candidates form
 * a tree (pruned Cartesian product of the heads' top-s lists) and a mask
 * lets each candidate attend only to its ancestors, so all paths are
 * verified in one forward pass.  Read here as ancestor-or-self; every node
 * also sees the whole KV-cache prefix of its sequence.
 *
 * Query row (b, h, t) -- sequence b, query head h, tree node t -- attends
 * to prefix keys p < prefix_len[b] of kv head h / (Hq / Hkv) and to the tree
 * keys of t's ancestors and t itself:
 *   out[b][h][t] = sum_j softmax_j(scale * q.k_j) v_j.
 *
 *   q           device [B][Hq][T][dh]     dtype (post-rotary queries)
 *   k_cache     device [B][Hkv][Lcap][dh] dtype
 *   v_cache     device [B][Hkv][Lcap][dh] dtype
 *   prefix_len  device [B] int32; values outside [0, Lcap] are clamped and
 *               flagged in the workspace's first int32 (nonzero = some value
 *               was clamped; written by every call, valid until the next
 *               call on the workspace)
 *   k_tree      device [B][Hkv][T][dh]    dtype (keys of the tree tokens)
 *   v_tree      device [B][Hkv][T][dh]    dtype
 *   parent      host [T] int32: parent[0] = -1, 0 <= parent[n] < n
 *   out         device [B][Hq][T][dh]     dtype
 *   mask_out    device [T][(T+63)/64] uint64 ancestor-or-self bit rows
 *               (bit j of word j/64 of row n), or NULL
 *
 * Limits: T <= 256, dh in {64, 128}, Hq % Hkv == 0, Lcap >= 0,
 * scale > 0; MEDUSA_ERR_SHAPE also when one kv head's query rows
 * (Hq/Hkv*T*dh elements) reach 4 GiB, when B*Hkv*Lcap*dh reaches 2^40, or
 * when the launch would need more than 2^31 - 1 workgroups (the workspace
 * size is then 0).  Arithmetic: MFMA (bf16 products, fp32
 * accumulation; fp32 MFMA in F32 mode), online softmax in fp32.
 * ---------------------------------------------------------------------- */
int tree_attention(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *prefix_len, const void *k_tree, const void *v_tree,
                   const int32_t *parent, int B, int Hq, int Hkv, int Lcap, int dh, int T,
                   float scale, int dtype, void *out, uint64_t *mask_out, void *ws,
                   size_t ws_bytes, void *stream);

size_t tree_attention_workspace_bytes(int B, int Hq, int Hkv, int Lcap, int dh, int T,
                                      int dtype);

/* ------------------------------------------------------------------------
 * tree_accept -- verify the candidates and keep the longest valid path.
 *
 * Node n > 0 carries token tok(n) = topk_ids[b][depth(n)-1][rank(n)], where
 * rank(n) is node_rank[n] or, when node_rank is NULL, the number of earlier
 * siblings of n.  Node c is checked against its parent's logits row
 * (logits[b][parent(c)]):
 *   MEDUSA_GREEDY  valid iff tok(c) is the row's argmax (equal maxima ->
 *                  smaller id): temperature-0 verification by argmax
 *                  comparison (explainer page, typical-acceptance section,
 *                  last paragraph);
 *   MEDUSA_TYPICAL p = softmax(row / temperature), H(p) = -sum p ln p,
 *                  valid iff p(tok) > min(eps, delta * exp(-H)) (same
 *                  section's inequality; its defaults eps = 0.09,
 *                  delta = 0.6).
 *   MEDUSA_TYPICAL_LOGLIK  as MEDUSA_TYPICAL; among equally deep valid
 *                  paths the one with the largest sum of ln p(tok) over its
 *                  nodes wins (page "Medusa：基于多Token预测的LLM推理加速",
 *                  section 5.3: its verification result carries such a
 *                  log-probability sum), then the lowest node index.
 *                  Scores are fp32.
 * The accepted path ends at the deepest node whose path from the root is
 * all valid (the first rejection ends a path); equal depths -> lowest
 * node index (MEDUSA_GREEDY, MEDUSA_TYPICAL).
 *
 *   logits          device [B][T][V] dtype (the base model's logits at every
 *                   tree node)
 *   topk_ids        device [B][K][s] int32 (from medusa_heads_topk)
 *   parent          host [T] int32 (as tree_attention)
 *   node_rank       host [T] int32 or NULL
 *   accept_len      device [B] int32: candidate tokens accepted, 0..K
 *   best_node       device [B] int32: last node of the accepted path
 *   accepted_tokens device [B][K] int32: tokens of the path, -1 padded
 *   node_tokens     device [B][T] int32 or NULL: tok(n), root = -1
 *   next_token      device [B] int32 or NULL: argmax of logits[b][best_node]
 *
 * Limits: T <= 256, depth <= K <= 16, rank < s <= 255, V >= 1; the typical
 * modes need temperature > 0, 0 < eps, 0 < delta.
 * ---------------------------------------------------------------------- */
int tree_accept(const void *logits, const int32_t *topk_ids, const int32_t *parent,
                const int32_t *node_rank, int B, int T, int V, int K, int s, int dtype, int mode,
                float temperature, float eps, float delta, int32_t *accept_len,
                int32_t *best_node, int32_t *accepted_tokens, int32_t *node_tokens,
                int32_t *next_token, void *ws, size_t ws_bytes, void *stream);

size_t tree_accept_workspace_bytes(int B, int T, int V, int K, int s);

/* ------------------------------------------------------------------------
 * medusa_sample_token -- a sampled bonus token from the best node's row.
 *
 * Sampled verification draws from p = softmax(row / temperature) (page
 * "Medusa：基于多Token预测的LLM推理加速", section 3.3; at temperature 0 it is
 * the argmax, which tree_accept's next_token already gives).  The draw is
 * the inversion of p's distribution function with a caller-supplied uniform:
 * token[b] is the first t whose cumulative probability P(<= t) exceeds
 * u[b].  The caller owns the random numbers, so equal inputs give equal
 * tokens.
 *
 *   logits  device [B][T][V] dtype (as tree_accept)
 *   rows    device [B] int32: the row of each sequence (e.g. tree_accept's
 *           best_node)
 *   u       device [B] float32 uniforms in [0, 1)
 *   token   device [B] int32: the drawn token; -1 when rows[b] is outside
 *           [0, T) or u[b] outside [0, 1)
 *
 * Arithmetic: fp32 (exp2 of the row minus its maximum, sums in a fixed
 * order), so a u within about 1e-6 of a cumulative boundary can land on
 * either neighbour.  Rows need at least one finite logit.  Limits: V >= 1,
 * temperature > 0.  Needs no workspace.
 * ---------------------------------------------------------------------- */
int medusa_sample_token(const void *logits, const int32_t *rows, const float *u, int B, int T,
                        int V, int dtype, float temperature, int32_t *token, void *stream);

/* ------------------------------------------------------------------------
 * tree_commit_kv -- append the accepted path's keys and values to the cache.
 *
 * The step after acceptance: the sequence grows by the root token and the
 * accepted candidates (page "Medusa：基于多Token预测的LLM推理加速", section 3.1,
 * step 4 of the decode loop; aiunderstanding page, section ディープダイブ: the
 * longest matching prefix is kept).  Their K/V rows already exist from the
 * tree pass: for each sequence b the rows of the nodes on the path
 * root -> best_node[b], in depth order, are copied to cache positions
 * prefix_len[b], prefix_len[b] + 1, ..., and prefix_len[b] advances by the
 * path length (depth(best) + 1 = accept_len + 1 rows).
 *
 *   k_cache, v_cache device [B][Hkv][Lcap][dh] dtype, updated in place
 *   prefix_len       device [B] int32, advanced in place
 *   k_tree, v_tree   device [B][Hkv][T][dh] dtype (as tree_attention)
 *   best_node        device [B] int32 (as written by tree_accept)
 *   parent           host [T] int32 (as tree_attention)
 *   committed        device [B] int32 or NULL: rows written for b; 0 when
 *                    the sequence was left untouched because prefix_len[b]
 *                    is outside [0, Lcap], best_node[b] is outside [0, T)
 *                    or the path does not fit below Lcap
 *
 * Limits: 1 <= T <= 256, dh * element size a multiple of 16 bytes.  A pure
 * copy (bit-exact).  Needs no workspace.
 * ---------------------------------------------------------------------- */
int tree_commit_kv(void *k_cache, void *v_cache, int32_t *prefix_len, const void *k_tree,
                   const void *v_tree, const int32_t *best_node, const int32_t *parent, int B,
                   int Hkv, int Lcap, int dh, int T, int dtype, int32_t *committed,
                   void *stream);

/* Text for a medusa_status value (static storage). */
const char *medusa_status_str(int status);

/* ABI version of this header (bumped on incompatible changes). */
int medusa_abi_version(void);

/* ------------------------------------------------------------------------
 * medusa_verify_forward -- the tree's verification logits from a forward
 * pass of N attention blocks and the LM head.
 *
 * Tree-attention section of the paper explainer page: all candidates are
 * verified in one forward pass under the tree mask; page
 * "Medusa：基于多Token预测的LLM推理加速", section 5.3, flattens the tree into
 * one sequence, runs the model once and reads the logits of every position.
 * The blocks here are attention-only (no MLP), pre-norm, without biases:
 *   x = rmsnorm(h) g_l (rounded to dtype), rmsnorm(h) = h / sqrt(mean(h^2) + eps)
 *   q = rope(x Wq_l^T), k = rope(x Wk_l^T), v = x Wv_l^T   (rounded to dtype)
 *   o = tree_attention(q, k_cache_l, v_cache_l, k, v) with scale 1/sqrt(dh)
 *   h = h + o Wo_l^T                                       (fp32)
 *   logits = (rmsnorm(h) g_final, rounded) W_lm^T          (fp32)
 * h starts as h0 (the tree tokens' embeddings).  rope rotates the pairs
 * (j, j + dh/2) of every head by pos * theta^(-2j/dh) with
 * pos = clamp(prefix_len[b], 0, Lcap) + depth(n): a node follows its
 * ancestors.  The caches hold keys already rotated at their positions.
 *
 *   h0          device [B][T][d] dtype
 *   g, wq, wk, wv, wo
 *               host arrays [N] of device pointers: g_l [d], wq_l [Hq*dh][d],
 *               wk_l and wv_l [Hkv*dh][d], wo_l [d][Hq*dh] (dtype, [out][in])
 *   g_final     device [d] dtype;  w_lm  device [V][d] dtype
 *   k_caches, v_caches
 *               host arrays [N] of device pointers, each [B][Hkv][Lcap][dh]
 *   prefix_len  device [B] int32 (as tree_attention); parent host [T] int32
 *   logits      device [B][T][V] float32
 *   hidden_out  device [B][T][d] float32 or NULL: h after the last block
 *   k_tree_out, v_tree_out
 *               device [N][B][Hkv][T][dh] dtype or NULL: every block's tree
 *               keys (rotated) and values, ready for tree_commit_kv
 *
 * Limits: 0 <= N <= 256, T <= 256, dh in {64, 128}, Hq % Hkv == 0,
 * d % 32 == 0 (BF16) or d % 16 == 0 (F32), B*T*V < 2^31, theta > 0,
 * eps >= 0.  Arithmetic: MFMA with fp32 accumulation, partial sums added
 * in a fixed order (results do not vary from run to run); rotary angles
 * in fp64.  Several kernels per block; the tree attention is the one
 * tree_attention runs.
 * ---------------------------------------------------------------------- */
int medusa_verify_forward(const void *h0, int N, const void *const *g, const void *const *wq,
                          const void *const *wk, const void *const *wv, const void *const *wo,
                          const void *g_final, const void *w_lm, const void *const *k_caches,
                          const void *const *v_caches, const int32_t *prefix_len,
                          const int32_t *parent, int B, int T, int d, int Hq, int Hkv, int dh,
                          int Lcap, int V, int dtype, double theta, float eps, float *logits,
                          float *hidden_out, void *k_tree_out, void *v_tree_out, void *ws,
                          size_t ws_bytes, void *stream);

size_t medusa_verify_forward_workspace_bytes(int B, int T, int d, int Hq, int Hkv, int dh,
                                             int Lcap, int V, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_VERIFY_H */
