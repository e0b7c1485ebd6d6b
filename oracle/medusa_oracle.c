/*
 * medusa_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, fp64 CPU reference of the Medusa verify step, used only to
 * check the HIP library: by tests/, by the package smoke check and by the
 * bench's CPU-baseline leg.  It shares no code, header or table with the HIP
 * path.  Every loop is the definition written out; the only liberty taken is
 * the order in which independent outputs are visited (and OpenMP over them).
 *
 * Sources (the Medusa pages): the paper explainer page "Medusa -- multiple
 * decoding heads" (sections: head architecture with its equation H_i and its
 * PyTorch head listing; tree attention with the ancestor-mask equation;
 * typical acceptance with its inequality and defaults; implementation notes
 * on s and the 63-node tree), the Chinese tutorial page (section 2.2 tree
 * mask construction, section 3.3 temperature-scaled distribution, section
 * 5.3 verification that stops at the first mismatch) and the aiunderstanding
 * page (accept the longest matching prefix).
 *
 * Readings where the pages are silent:
 *  - weights are [out][in] (torch Linear); no biases.
 *  - bf16 mode: one rounding point, z = SiLU(W1 h) + h is rounded to bf16
 *    (nearest-even) from its fp32 value before W2; logits are not rounded.
 *  - top-s order: larger logit first, equal logits -> smaller token id.
 *  - the tree mask is ancestor-or-self; every node sees the whole prefix.
 *  - GQA: query head h reads kv head h / (Hq / Hkv).
 *  - node c is verified against its parent's logits row.
 *  - typical: p = softmax(logits / temperature), H in nats, strict ">".
 *  - among equally long valid paths the lowest node index wins.
 *  - greedy argmax ties -> smallest token id.
 *
 * Parity status: every entry point here is pinned by tests in
 * tests/test_oracle_pins.py (brute force, closed forms, hand-computed cases).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG -1
#define OR_ERR_TREE -2

/* ---------------------------------------------------------------- values */

/* dtype 0: IEEE fp32 array; dtype 1: bf16 bit patterns (upper half of fp32). */
static double ld(const void *p, size_t i, int dtype)
{
    if (dtype == 0)
        return (double)((const float *)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Round an fp32 value to the nearest bf16 value, ties to even mantissa. */
static float round_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u = (u + 0x7FFFu + lsb) & 0xFFFF0000u;
    float r;
    memcpy(&r, &u, sizeof r);
    return r;
}

/* "a ranks before b" for candidate lists: larger value, then smaller id. */
static int ranks_before(double va, int ia, double vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

/* ------------------------------------------------------------------ heads */

/*
 * H_i(h) = W2_i (SiLU(W1_i h) + h), SiLU(x) = x * sigmoid(x), for every
 * sequence b and head i, then the s best token ids of each logits vector.
 * (Head equation and the bias-free two-Linear listing on the explainer page.)
 *
 * hidden [B][d], w1 [K][d][d], w2 [K][V][d], stored as dtype.
 * Outputs (any may be NULL except topk_ids):
 *   z_out [B][K][d]   the W2 input (after the bf16 rounding in bf16 mode)
 *   logits [B][K][V]  fp64 logits
 *   topk_ids, topk_vals [B][K][s]
 */
int oracle_heads_topk(const void *hidden, const void *w1, const void *w2,
                      int B, int K, int d, int V, int s, int dtype,
                      double *z_out, double *logits, int32_t *topk_ids,
                      double *topk_vals)
{
    if (!hidden || !w1 || !w2 || !topk_ids || B < 1 || K < 1 || d < 1 || V < 1 || s < 1 ||
        s > V || (dtype != 0 && dtype != 1))
        return OR_ERR_ARG;

    double *z = (double *)malloc(sizeof(double) * (size_t)B * K * d);
    double *lg = logits ? logits : (double *)malloc(sizeof(double) * (size_t)B * K * V);
    if (!z || !lg) {
        free(z);
        if (!logits) free(lg);
        return OR_ERR_ARG;
    }

    /* stage 1: u = W1_i h ; z = SiLU(u) + h */
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < K; ++i) {
#pragma omp parallel for schedule(static)
            for (int j = 0; j < d; ++j) {
                double u = 0.0;
                const size_t row = ((size_t)i * d + j) * (size_t)d;
                for (int k = 0; k < d; ++k)
                    u += ld(w1, row + k, dtype) * ld(hidden, (size_t)b * d + k, dtype);
                double silu = u / (1.0 + exp(-u));
                double zj = silu + ld(hidden, (size_t)b * d + j, dtype);
                if (dtype == 1)
                    zj = (double)round_to_bf16((float)zj);
                z[((size_t)b * K + i) * d + j] = zj;
            }
        }

    /* stage 2: logits_v = W2_i[v] . z  (each W2 row visited once for all b) */
    for (int i = 0; i < K; ++i) {
#pragma omp parallel for schedule(static)
        for (int v = 0; v < V; ++v) {
            const size_t row = ((size_t)i * V + v) * (size_t)d;
            for (int b = 0; b < B; ++b) {
                const double *zb = z + ((size_t)b * K + i) * d;
                double acc = 0.0;
                for (int j = 0; j < d; ++j)
                    acc += ld(w2, row + j, dtype) * zb[j];
                lg[((size_t)b * K + i) * V + v] = acc;
            }
        }
    }

    /* top-s: s rounds of "best not yet taken" */
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < K; ++i) {
            const double *row = lg + ((size_t)b * K + i) * V;
            int32_t *ids = topk_ids + ((size_t)b * K + i) * s;
            for (int r = 0; r < s; ++r) {
                int best = -1;
                for (int v = 0; v < V; ++v) {
                    int taken = 0;
                    for (int q = 0; q < r; ++q)
                        if (ids[q] == v) taken = 1;
                    if (taken) continue;
                    if (best < 0 || ranks_before(row[v], v, row[best], best))
                        best = v;
                }
                ids[r] = best;
                if (topk_vals)
                    topk_vals[((size_t)b * K + i) * s + r] = row[best];
            }
        }

    if (z_out)
        memcpy(z_out, z, sizeof(double) * (size_t)B * K * d);
    free(z);
    if (!logits) free(lg);
    return OR_OK;
}

/* ------------------------------------------------------------------- tree */

/*
 * Tree structure from a parent array in canonical order (parents before
 * children, parent[0] = -1).  depth(root) = 0, depth(n) = depth(parent)+1;
 * rank(n) = node_rank[n] if given, else the number of earlier siblings.
 * mask row n (words of 64 bits, bit j of word j/64) holds n and all its
 * ancestors (the tree-attention mask equation, read as ancestor-or-self).
 * Checks: depth <= K, rank < s.  Any output may be NULL.
 */
int oracle_tree(const int32_t *parent, const int32_t *node_rank, int T, int K, int s,
                int32_t *depth, int32_t *rank, uint64_t *mask)
{
    if (!parent || T < 1 || K < 0 || s < 1)
        return OR_ERR_ARG;
    if (parent[0] != -1)
        return OR_ERR_TREE;
    for (int n = 1; n < T; ++n)
        if (parent[n] < 0 || parent[n] >= n)
            return OR_ERR_TREE;
    const int W = (T + 63) / 64;
    for (int n = 0; n < T; ++n) {
        int dn = 0;
        for (int a = n; parent[a] >= 0; a = parent[a])
            ++dn;
        int rn = 0;
        if (n > 0) {
            if (node_rank) {
                rn = node_rank[n];
            } else {
                for (int m = 1; m < n; ++m)
                    if (parent[m] == parent[n]) ++rn;
            }
        }
        if (dn > K || rn < 0 || (n > 0 && rn >= s))
            return OR_ERR_TREE;
        if (depth) depth[n] = dn;
        if (rank) rank[n] = rn;
        if (mask) {
            uint64_t *row = mask + (size_t)n * W;
            for (int w = 0; w < W; ++w) row[w] = 0;
            for (int a = n; a >= 0; a = parent[a])
                row[a / 64] |= (uint64_t)1 << (a % 64);
        }
    }
    if (node_rank) {
        /* two siblings may not claim the same candidate rank */
        for (int n = 1; n < T; ++n)
            for (int m = 1; m < n; ++m)
                if (parent[m] == parent[n] && node_rank[m] == node_rank[n])
                    return OR_ERR_TREE;
    }
    return OR_OK;
}

/* -------------------------------------------------------------- attention */

/*
 * Tree attention for selected output rows.  Query row (b, h, t) attends to
 * every prefix key p < prefix_len[b] of kv head h/(Hq/Hkv) and to the tree
 * keys j that are ancestors of t or t itself; scores scale * q.k, softmax,
 * weighted sum of values (tree-attention section of the explainer page: one
 * pass, each candidate sees only its own ancestors).
 *
 * q [B][Hq][T][dh]; k_cache, v_cache [B][Hkv][Lcap][dh];
 * k_tree, v_tree [B][Hkv][T][dh]; prefix_len [B] (clamped to [0, Lcap]).
 * rows: nrows triples (b, h, t), or NULL for all B*Hq*T rows in order.
 * out: [nrows][dh] fp64.
 */
int oracle_tree_attention(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *prefix_len, const void *k_tree, const void *v_tree,
                          const int32_t *parent, int B, int Hq, int Hkv, int Lcap, int dh,
                          int T, double scale, int dtype, const int32_t *rows, int nrows,
                          double *out)
{
    if (!q || !k_cache || !v_cache || !prefix_len || !k_tree || !v_tree || !parent || !out ||
        B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Lcap < 0 || dh < 1 || T < 1 ||
        (dtype != 0 && dtype != 1))
        return OR_ERR_ARG;
    if (oracle_tree(parent, NULL, T, T, T, NULL, NULL, NULL) != OR_OK)
        return OR_ERR_TREE;
    const int G = Hq / Hkv;
    const int total = rows ? nrows : B * Hq * T;

#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < total; ++r) {
        int b, h, t;
        if (rows) {
            b = rows[3 * r];
            h = rows[3 * r + 1];
            t = rows[3 * r + 2];
        } else {
            b = r / (Hq * T);
            h = (r / T) % Hq;
            t = r % T;
        }
        double *o = out + (size_t)r * dh;
        if (b < 0 || b >= B || h < 0 || h >= Hq || t < 0 || t >= T) {
            for (int e = 0; e < dh; ++e) o[e] = NAN;
            continue;
        }
        const int kvh = h / G;
        int L = prefix_len[b];
        if (L < 0) L = 0;
        if (L > Lcap) L = Lcap;
        const size_t qoff = (((size_t)b * Hq + h) * T + t) * dh;
        const size_t coff = ((size_t)b * Hkv + kvh) * (size_t)Lcap * dh;
        const size_t toff = ((size_t)b * Hkv + kvh) * (size_t)T * dh;

        /* visible tree keys: t and its ancestors */
        int *anc = (int *)malloc(sizeof(int) * (size_t)T);
        int na = 0;
        for (int a = t; a >= 0; a = parent[a])
            anc[na++] = a;

        const int nkeys = L + na;
        double *sc = (double *)malloc(sizeof(double) * (size_t)(nkeys > 0 ? nkeys : 1));
        double m = -INFINITY;
        for (int p = 0; p < L; ++p) {
            double acc = 0.0;
            for (int e = 0; e < dh; ++e)
                acc += ld(q, qoff + e, dtype) * ld(k_cache, coff + (size_t)p * dh + e, dtype);
            sc[p] = scale * acc;
            if (sc[p] > m) m = sc[p];
        }
        for (int a = 0; a < na; ++a) {
            double acc = 0.0;
            for (int e = 0; e < dh; ++e)
                acc += ld(q, qoff + e, dtype) * ld(k_tree, toff + (size_t)anc[a] * dh + e, dtype);
            sc[L + a] = scale * acc;
            if (sc[L + a] > m) m = sc[L + a];
        }
        double den = 0.0;
        for (int k = 0; k < nkeys; ++k) {
            sc[k] = exp(sc[k] - m);
            den += sc[k];
        }
        /* o[e] = sum over the visible keys in the order prefix 0..L-1, then
           the ancestors; the key loop is outside so that each V row is read
           once (each o[e] still sums its terms in that same order) */
        for (int e = 0; e < dh; ++e)
            o[e] = 0.0;
        for (int p = 0; p < L; ++p)
            for (int e = 0; e < dh; ++e)
                o[e] += sc[p] * ld(v_cache, coff + (size_t)p * dh + e, dtype);
        for (int a = 0; a < na; ++a)
            for (int e = 0; e < dh; ++e)
                o[e] += sc[L + a] * ld(v_tree, toff + (size_t)anc[a] * dh + e, dtype);
        for (int e = 0; e < dh; ++e)
            o[e] /= den;
        free(sc);
        free(anc);
    }
    return OR_OK;
}

/* ------------------------------------------------------------- acceptance */

/*
 * Verification of the candidate tree and choice of the longest valid path.
 *
 * Node n > 0 carries token tok(n) = topk_ids[b][depth(n)-1][rank(n)] and is
 * checked against the logits row of its parent:
 *  greedy (mode 0): valid iff tok(n) is the row's argmax (ties -> smaller
 *    id) -- temperature-0 verification by argmax comparison;
 *  typical (mode 1): p = softmax(row / temperature); H = -sum p ln p;
 *    valid iff p(tok) > min(eps, delta * exp(-H)) -- the typical-acceptance
 *    inequality with its defaults eps = 0.09, delta = 0.6.
 * A node is reachable when it and every ancestor below the root are valid;
 * the accepted path ends at the deepest reachable node (lowest index among
 * equals), verification stopping at the first mismatch along each path.
 *
 * logits [B][T][V] (dtype), topk_ids [B][K][s], parent [T], node_rank [T] or
 * NULL.  Outputs: accept_len [B], best_node [B], accepted_tokens [B][K]
 * (-1 padded), node_tokens [B][T] (root -1) or NULL, next_token [B] (argmax
 * of the best node's row) or NULL, valid [B][T] or NULL, ratio [B][T]
 * (typical: p/threshold of each node, greedy: 1 if valid else 0) or NULL,
 * entropy [B][T] (H of each row in typical mode) or NULL.
 */
int oracle_tree_accept(const void *logits, const int32_t *topk_ids, const int32_t *parent,
                       const int32_t *node_rank, int B, int T, int V, int K, int s, int dtype,
                       int mode, double temperature, double eps, double delta,
                       int32_t *accept_len, int32_t *best_node, int32_t *accepted_tokens,
                       int32_t *node_tokens, int32_t *next_token, uint8_t *valid_out,
                       double *ratio_out, double *entropy_out, double *score_out)
{
    if (!logits || !topk_ids || !parent || !accept_len || !best_node || !accepted_tokens ||
        B < 1 || T < 1 || V < 1 || K < 0 || s < 1 || (dtype != 0 && dtype != 1) ||
        (mode != 0 && mode != 1 && mode != 2))
        return OR_ERR_ARG;
    if (mode != 0 && !(temperature > 0.0))
        return OR_ERR_ARG;
    int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * T);
    int32_t *rank = (int32_t *)malloc(sizeof(int32_t) * T);
    int st = oracle_tree(parent, node_rank, T, K, s, depth, rank, NULL);
    if (st != OR_OK) {
        free(depth);
        free(rank);
        return st;
    }

#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * T);
        uint8_t *valid = (uint8_t *)malloc(T);
        double *prob = (double *)malloc(sizeof(double) * V);
        double *lp = (double *)malloc(sizeof(double) * T);   /* ln p of each node's token */
        tok[0] = -1;
        for (int n = 0; n < T; ++n) lp[n] = 0.0;
        for (int n = 1; n < T; ++n)
            tok[n] = topk_ids[((size_t)b * K + depth[n] - 1) * s + rank[n]];
        valid[0] = 1;
        if (ratio_out) ratio_out[(size_t)b * T] = 0.0;
        for (int n = 0; n < T; ++n)
            if (entropy_out) entropy_out[(size_t)b * T + n] = NAN;

        for (int p = 0; p < T; ++p) {
            int has_child = 0;
            for (int c = p + 1; c < T; ++c)
                if (parent[c] == p) has_child = 1;
            if (!has_child) continue;
            const size_t roff = ((size_t)b * T + p) * V;
            if (mode == 0) {
                int am = 0;
                for (int v = 1; v < V; ++v)
                    if (ld(logits, roff + v, dtype) > ld(logits, roff + am, dtype)) am = v;
                for (int c = p + 1; c < T; ++c)
                    if (parent[c] == p) {
                        valid[c] = (tok[c] == am);
                        if (ratio_out) ratio_out[(size_t)b * T + c] = valid[c] ? 1.0 : 0.0;
                    }
            } else {
                double mx = -INFINITY;
                for (int v = 0; v < V; ++v) {
                    double zv = ld(logits, roff + v, dtype) / temperature;
                    prob[v] = zv;
                    if (zv > mx) mx = zv;
                }
                double den = 0.0;
                for (int v = 0; v < V; ++v) {
                    prob[v] = exp(prob[v] - mx);
                    den += prob[v];
                }
                double H = 0.0;
                for (int v = 0; v < V; ++v) {
                    prob[v] /= den;
                    if (prob[v] > 0.0) H -= prob[v] * log(prob[v]);
                }
                double thr = delta * exp(-H);
                if (eps < thr) thr = eps;
                if (entropy_out) entropy_out[(size_t)b * T + p] = H;
                for (int c = p + 1; c < T; ++c)
                    if (parent[c] == p) {
                        double pc = (tok[c] >= 0 && tok[c] < V) ? prob[tok[c]] : 0.0;
                        valid[c] = pc > thr;
                        lp[c] = pc > 0.0 ? log(pc) : -INFINITY;
                        if (ratio_out) ratio_out[(size_t)b * T + c] = pc / thr;
                    }
            }
        }

        /* longest valid path: walk every node up to the root.  Equal depths:
           mode 2 prefers the larger path log-likelihood (sum of ln p of the
           path's tokens), then the lower index; modes 0 and 1 the lower index. */
        int best = 0, best_d = 0;
        double best_s = 0.0;
        if (score_out) score_out[(size_t)b * T] = 0.0;
        for (int n = 1; n < T; ++n) {
            int ok = 1;
            double sc = 0.0;
            for (int a = n; a > 0; a = parent[a]) {
                if (!valid[a]) ok = 0;
                sc += lp[a];
            }
            if (score_out) score_out[(size_t)b * T + n] = sc;
            if (ok && (depth[n] > best_d || (mode == 2 && depth[n] == best_d && sc > best_s))) {
                best = n;
                best_d = depth[n];
                best_s = sc;
            }
        }
        accept_len[b] = best_d;
        best_node[b] = best;
        for (int k = 0; k < K; ++k)
            accepted_tokens[(size_t)b * K + k] = -1;
        for (int a = best; a > 0; a = parent[a])
            accepted_tokens[(size_t)b * K + depth[a] - 1] = tok[a];
        if (node_tokens)
            for (int n = 0; n < T; ++n) node_tokens[(size_t)b * T + n] = tok[n];
        if (valid_out)
            for (int n = 0; n < T; ++n) valid_out[(size_t)b * T + n] = valid[n];
        if (next_token) {
            const size_t roff = ((size_t)b * T + best) * V;
            int am = 0;
            for (int v = 1; v < V; ++v)
                if (ld(logits, roff + v, dtype) > ld(logits, roff + am, dtype)) am = v;
            next_token[b] = am;
        }
        free(tok);
        free(valid);
        free(prob);
        free(lp);
    }
    free(depth);
    free(rank);
    return OR_OK;
}

/* Threads OpenMP will use (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif
