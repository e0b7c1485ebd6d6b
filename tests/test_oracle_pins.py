"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against a library routine, a closed form, a
brute-force restatement or a hand-derived case, chosen so that a plausible
mistake (a dropped residual, a ReLU for the SiLU, a transposed weight, a
mask without self, a wrong tie-break, a missing temperature) fails one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from medusa_tree_verification_amd import workloads as W
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- heads
def test_heads_w1_zero_is_plain_gemv():
    """W1 = 0 makes SiLU(0) + h = h, so logits = W2 h (numpy GEMV)."""
    rng = np.random.default_rng(1)
    B, K, d, V, s = 2, 3, 32, 50, 4
    h = rng.standard_normal((B, d)).astype(np.float32)
    w1 = np.zeros((K, d, d), np.float32)
    w2 = rng.standard_normal((K, V, d)).astype(np.float32)
    out = oracle.heads_topk(h, w1, w2, s, "f32")
    ref = np.einsum("kvd,bd->bkv", w2.astype(np.float64), h.astype(np.float64))
    np.testing.assert_allclose(out["logits"], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(out["z"], np.broadcast_to(h[:, None, :], (B, K, d)))


def test_heads_silu_and_residual_closed_forms():
    """W1 = c*I gives u = c h.  With SiLU(x) = x*sigmoid(x):
    z(h) - z(-h) = c h + 2 h   (odd part of SiLU is x/2, plus the residual)
    z(h) + z(-h) = c h tanh(c h / 2)   (even part)."""
    rng = np.random.default_rng(2)
    d, c = 16, 0.75
    h = rng.standard_normal(d).astype(np.float32) * 3
    hb = np.stack([h, -h])
    w1 = (c * np.eye(d, dtype=np.float32))[None]
    w2 = np.eye(d, dtype=np.float32)[None]  # logits = z
    out = oracle.heads_topk(hb, w1, w2, 1, "f32")
    z = out["z"][:, 0, :]
    x = c * h.astype(np.float64)
    np.testing.assert_allclose(z[0] - z[1], x + 2 * h, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(z[0] + z[1], x * np.tanh(x / 2), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(out["logits"][:, 0, :], z, rtol=0, atol=0)


def test_heads_weight_orientation_out_in():
    """torch Linear convention [out][in]: W1[j][k] = 1 makes u_j = h_k, and
    W2[v][j] = 1 makes logit_v = z_j."""
    d, V = 8, 5
    h = np.arange(1, d + 1, dtype=np.float32)
    w1 = np.zeros((1, d, d), np.float32)
    w1[0, 2, 6] = 1.0  # u_2 = h_6 = 7
    w2 = np.zeros((1, V, d), np.float32)
    w2[0, 4, 2] = 1.0  # logit_4 = z_2
    out = oracle.heads_topk(h[None], w1, w2, 1, "f32")
    z = out["z"][0, 0]
    u2 = 7.0
    assert abs(z[2] - (u2 / (1 + math.exp(-u2)) + 3.0)) < 1e-12
    others = np.delete(np.arange(d), 2)
    np.testing.assert_array_equal(z[others], h[others])  # SiLU(0) = 0
    assert out["logits"][0, 0, 4] == z[2]
    assert out["topk_ids"][0, 0, 0] == 4


def test_heads_topk_matches_sort_with_ties():
    """Top-s = first s of a stable sort by (value desc, id asc); ties planted."""
    rng = np.random.default_rng(3)
    B, K, d, V, s = 3, 2, 8, 40, 6
    h = np.zeros((B, d), np.float32)
    h[:, 0] = 1.0
    w1 = np.zeros((K, d, d), np.float32)
    # logits = W2[:, :, 0] exactly; use small integers so ties are exact
    w2 = np.zeros((K, V, d), np.float32)
    w2[:, :, 0] = rng.integers(-3, 4, size=(K, V)).astype(np.float32)
    out = oracle.heads_topk(h, w1, w2, s, "f32")
    for b in range(B):
        for k in range(K):
            row = w2[k, :, 0].astype(np.float64)
            order = np.lexsort((np.arange(V), -row))[:s]
            np.testing.assert_array_equal(out["topk_ids"][b, k], order)
            np.testing.assert_array_equal(out["topk_vals"][b, k], row[order])


def test_heads_bf16_single_rounding_point():
    """bf16 mode rounds z once (fp64 -> fp32 -> bf16, nearest-even, checked
    with torch's own conversion) and keeps logits unrounded (= W2 z)."""
    rng = np.random.default_rng(4)
    B, K, d, V, s = 2, 2, 64, 30, 3
    hb = W.encode(rng.standard_normal((B, d)), W.BF16)
    w1b = W.encode(rng.standard_normal((K, d, d)) * 0.1, W.BF16)
    w2b = W.encode(rng.standard_normal((K, V, d)) * 0.1, W.BF16)
    ob = oracle.heads_topk(hb, w1b, w2b, s, "bf16")
    # same values in fp32 mode: unrounded z
    of = oracle.heads_topk(W.decode(hb, W.BF16).astype(np.float32),
                           W.decode(w1b, W.BF16).astype(np.float32),
                           W.decode(w2b, W.BF16).astype(np.float32), s, "f32")
    z_ref = torch.from_numpy(of["z"].astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(ob["z"], z_ref)
    assert not np.array_equal(of["z"], ob["z"])  # the rounding point exists
    w2d = W.decode(w2b, W.BF16)
    np.testing.assert_allclose(ob["logits"], np.einsum("kvd,bkd->bkv", w2d, ob["z"]),
                               rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ tree
@pytest.mark.parametrize("K,s,T", [(3, 2, 15), (4, 3, 121), (2, 3, 13), (1, 1, 2)])
def test_full_product_counts(K, s, T):
    """The uncut product has sum_{j<=K} s^j nodes (k=4, s=3: 81 leaf paths)."""
    t = W.full_product_tree(K, s)
    assert t.T == T == sum(s ** j for j in range(K + 1))
    o = oracle.tree(t.parent, K, s)
    assert np.bincount(o["depth"]).tolist() == [s ** j for j in range(K + 1)]
    assert int((o["depth"] == K).sum()) == s ** K


def test_default_pruned_trees():
    """63 candidates + root for the 4-head tree; 255 + root for 5 heads."""
    t64 = W.pruned_tree(W.WORKLOADS["llama7b_b1"].rates, 3, 64)
    assert np.bincount(oracle.tree(t64.parent, 4, 3)["depth"]).tolist() == [1, 3, 9, 25, 26]
    t256 = W.pruned_tree(W.WORKLOADS["large_vocab_typical"].rates, 3, 256)
    assert np.bincount(oracle.tree(t256.parent, 5, 3)["depth"]).tolist() == [1, 3, 9, 27, 81, 135]


def _trees():
    out = [W.full_product_tree(3, 2), W.full_product_tree(4, 3), W.chain_tree(5),
           W.pruned_tree(W.WORKLOADS["llama7b_b1"].rates, 3, 64),
           W.pruned_tree(W.WORKLOADS["large_vocab_typical"].rates, 3, 256),
           W.tree_from_paths([()])]
    out += [W.random_tree(100 + i, T, 6, 4) for i, T in enumerate([2, 7, 33, 65, 129])]
    return out


@pytest.mark.parametrize("ti", range(11))
def test_tree_mask_and_ranks_against_rank_tuples(ti):
    """Mask row n = ancestors-or-self of n, found independently from the
    rank tuples (prefix relation); rank = last tuple entry; depth = length."""
    t = _trees()[ti]
    K = max(len(p) for p in t.paths)
    s = max([p[-1] for p in t.paths if p] + [0]) + 1
    o = oracle.tree(t.parent, K, s)
    T = t.T
    for n in range(T):
        assert o["depth"][n] == len(t.paths[n])
        if n:
            assert o["rank"][n] == t.paths[n][-1]
        bits = set(j for j in range(T) if (int(o["mask"][n, j // 64]) >> (j % 64)) & 1)
        ref = set(m for m in range(T) if brute.is_prefix(t.paths[m], t.paths[n]))
        assert bits == ref
        assert len(bits) == len(t.paths[n]) + 1          # popcount = depth + 1
        assert max(bits) == n                           # lower-triangular, self included
        if n:
            pbits = set(j for j in range(T)
                        if (int(o["mask"][t.parent[n], j // 64]) >> (j % 64)) & 1)
            assert bits == pbits | {n}                  # mask(n) = {n} U mask(parent)


def test_tree_rejects_bad_parent_arrays():
    with pytest.raises(oracle.OracleError):
        oracle.tree(np.array([0, 0], np.int32), 2, 2)      # root must be -1
    with pytest.raises(oracle.OracleError):
        oracle.tree(np.array([-1, 1], np.int32), 2, 2)     # not parent-before-child
    with pytest.raises(oracle.OracleError):
        oracle.tree(np.array([-1, 0, 1, 2], np.int32), 2, 2)  # depth 3 > K
    with pytest.raises(oracle.OracleError):
        oracle.tree(np.array([-1, 0, 0, 0], np.int32), 3, 2)  # rank 2 >= s
    with pytest.raises(oracle.OracleError):
        oracle.tree(np.array([-1, 0, 0], np.int32), 2, 2, node_rank=np.array([0, 1, 1]))


# ------------------------------------------------------------- attention
def _attn_inputs(seed, B, Hq, Hkv, T, dh, Lcap, L):
    rng = np.random.default_rng(seed)
    f = lambda *sh: rng.standard_normal(sh).astype(np.float32)
    return dict(q=f(B, Hq, T, dh), k_cache=f(B, Hkv, Lcap, dh), v_cache=f(B, Hkv, Lcap, dh),
                k_tree=f(B, Hkv, T, dh), v_tree=f(B, Hkv, T, dh),
                prefix_len=np.asarray(L, np.int32))


@pytest.mark.parametrize("tree_kind", ["full", "random", "pruned"])
def test_attention_equals_per_path_causal_attention(tree_kind):
    """Tree-masked attention of node t == ordinary causal attention over the
    flat sequence prefix + (root..t path), read at its last position: what the
    tree mask buys is verifying every path in one pass."""
    if tree_kind == "full":
        t = W.full_product_tree(3, 2)
    elif tree_kind == "random":
        t = W.random_tree(7, 20, 5, 3)
    else:
        t = W.pruned_tree(W.WORKLOADS["llama7b_b1"].rates, 3, 64)
    B, Hq, Hkv, dh, Lcap = 2, 4, 2, 8, 9
    L = [9, 4]
    x = _attn_inputs(11, B, Hq, Hkv, t.T, dh, Lcap, L)
    scale = 1 / math.sqrt(dh)
    out = oracle.tree_attention(**x, parent=t.parent, scale=scale, dtype="f32")
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            for n in range(t.T):
                path = brute.path_nodes(t.paths, n)
                ks = np.concatenate([x["k_cache"][b, kv, :L[b]], x["k_tree"][b, kv, path]])
                vs = np.concatenate([x["v_cache"][b, kv, :L[b]], x["v_tree"][b, kv, path]])
                qs = np.concatenate([np.zeros((L[b], dh)), x["q"][b, h, path]])  # only last row used
                ref = brute.causal_attention_last(qs.astype(np.float64), ks.astype(np.float64),
                                                  vs.astype(np.float64), scale)
                np.testing.assert_allclose(out[b, h, n], ref, rtol=1e-10, atol=1e-12)


def test_attention_chain_tree_is_causal_sdpa():
    """A chain tree (s = 1) is plain causal attention: torch SDPA, fp64."""
    K, dh, L = 6, 16, 11
    t = W.chain_tree(K)
    x = _attn_inputs(12, 1, 2, 2, t.T, dh, L, [L])
    out = oracle.tree_attention(**x, parent=t.parent, scale=1 / math.sqrt(dh), dtype="f32")
    for h in range(2):
        k = np.concatenate([x["k_cache"][0, h], x["k_tree"][0, h]]).astype(np.float64)
        v = np.concatenate([x["v_cache"][0, h], x["v_tree"][0, h]]).astype(np.float64)
        q = np.concatenate([np.zeros((L, dh)), x["q"][0, h]]).astype(np.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            is_causal=True)[0, L:].numpy()
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-10, atol=1e-12)


def test_attention_single_node_is_decode_attention():
    """T = 1: one query over prefix + itself (torch SDPA, no mask)."""
    dh, L = 32, 40
    x = _attn_inputs(13, 1, 1, 1, 1, dh, L, [L])
    out = oracle.tree_attention(**x, parent=np.array([-1], np.int32), scale=0.3, dtype="f32")
    k = np.concatenate([x["k_cache"][0, 0], x["k_tree"][0, 0]]).astype(np.float64)
    v = np.concatenate([x["v_cache"][0, 0], x["v_tree"][0, 0]]).astype(np.float64)
    q = x["q"][0, 0].astype(np.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=0.3)[0].numpy()
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-10, atol=1e-12)


def test_attention_closed_forms():
    """q = 0 -> mean of the visible v rows; all v equal -> that row;
    prefix length 0 -> ancestors only; prefix longer than the cache is clamped."""
    t = W.full_product_tree(2, 3)
    dh, Lcap = 8, 5
    x = _attn_inputs(14, 3, 2, 2, t.T, dh, Lcap, [5, 0, 99])
    x["q"][:] = 0
    out = oracle.tree_attention(**x, parent=t.parent, scale=0.5, dtype="f32")
    for b, L in enumerate([5, 0, 5]):
        for n in range(t.T):
            path = brute.path_nodes(t.paths, n)
            vis = np.concatenate([x["v_cache"][b, 0, :L], x["v_tree"][b, 0, path]])
            np.testing.assert_allclose(out[b, 0, n], vis.astype(np.float64).mean(0), rtol=1e-12,
                                       atol=1e-12)
    y = _attn_inputs(15, 1, 1, 1, t.T, dh, Lcap, [3])
    y["v_cache"][:] = y["v_tree"][:] = np.arange(dh, dtype=np.float32)
    out = oracle.tree_attention(**y, parent=t.parent, scale=0.5, dtype="f32")
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(np.arange(dh), (t.T, dh)), rtol=1e-12)


def test_attention_rows_subset_matches_full():
    t = W.full_product_tree(2, 2)
    x = _attn_inputs(16, 2, 4, 2, t.T, 8, 6, [6, 3])
    full = oracle.tree_attention(**x, parent=t.parent, scale=0.35, dtype="f32")
    rows = np.array([[1, 3, 6], [0, 0, 0], [1, 1, 2]], np.int32)
    sub = oracle.tree_attention(**x, parent=t.parent, scale=0.35, dtype="f32", rows=rows)
    for i, (b, h, n) in enumerate(rows):
        np.testing.assert_array_equal(sub[i], full[b, h, n])


# ------------------------------------------------------------ acceptance
def test_typical_hand_cases():
    g = json.load(open(os.path.join(GOLDEN, "typical_acceptance_cases.json")))
    for c in g["cases"]:
        p = np.array(c["p"], np.float64)
        V = len(p)
        logits = np.where(p > 0, np.log(np.maximum(p, 1e-300)), -1e4).astype(np.float32)
        # root with V children at depth 1; child r carries token r
        parent = np.array([-1] + [0] * V, np.int32)
        ids = np.arange(V, dtype=np.int32).reshape(1, 1, V)
        L = np.zeros((1, V + 1, V), np.float32)
        L[0, 0] = logits
        o = oracle.tree_accept(L, ids, parent, "f32", "typical", temperature=1.0,
                               eps=g["eps"], delta=g["delta"])
        acc = [r for r in range(V) if o["valid"][0, 1 + r]]
        assert acc == c["accepted"], c["name"]
        assert abs(o["entropy"][0, 0] - c["H"]) < 1e-6, c["name"]
        thr = min(g["eps"], g["delta"] * math.exp(-o["entropy"][0, 0]))
        assert abs(thr - c["threshold"]) < 1e-6, c["name"]
        assert o["accept_len"][0] == (1 if acc else 0)
        assert o["best_node"][0] == (1 + acc[0] if acc else 0)


def test_typical_temperature_scales_logits():
    """softmax(logits / T): logits 2*ln p at T = 2 gives back p."""
    p = np.array([0.7, 0.2, 0.06, 0.04])
    parent = np.array([-1, 0, 0, 0, 0], np.int32)
    ids = np.arange(4, dtype=np.int32).reshape(1, 1, 4)
    L = np.zeros((1, 5, 4), np.float32)
    L[0, 0] = 2 * np.log(p)
    o = oracle.tree_accept(L, ids, parent, "f32", "typical", temperature=2.0)
    assert [r for r in range(4) if o["valid"][0, 1 + r]] == [0, 1]
    assert abs(o["entropy"][0, 0] - 0.86912) < 1e-5
    o1 = oracle.tree_accept(L, ids, parent, "f32", "typical", temperature=1.0)
    assert o1["entropy"][0, 0] < 0.8  # sharper at T = 1


def test_greedy_argmax_and_ties():
    """Greedy: child valid iff its token is the parent row's argmax; equal
    maxima resolve to the smaller token id."""
    parent = np.array([-1, 0, 0, 0], np.int32)
    ids = np.array([[[5, 2, 7]]], np.int32)
    L = np.zeros((1, 4, 8), np.float32)
    L[0, 0, [2, 5]] = 3.0   # tie between tokens 2 and 5 -> 2
    o = oracle.tree_accept(L, ids, parent, "f32", "greedy")
    assert o["valid"][0].tolist() == [1, 0, 1, 0]
    assert o["accept_len"][0] == 1 and o["best_node"][0] == 2
    assert o["accepted_tokens"][0].tolist() == [2]
    assert o["next_token"][0] == 0  # leaf row all zeros -> token 0


def test_stop_at_first_failure_on_a_chain():
    """Verification along a path stops at the first rejected token."""
    t = W.chain_tree(4)
    ids = np.array([[[3], [1], [4], [1]]], np.int32)
    L = np.zeros((1, 5, 6), np.float32)
    for n, tok in enumerate([3, 1, 0, 1]):   # depth-3 candidate 4 is not the argmax
        L[0, n, tok] = 1.0
    o = oracle.tree_accept(L, ids, t.parent, "f32", "greedy")
    assert o["valid"][0].tolist() == [1, 1, 1, 0, 1]
    assert o["accept_len"][0] == 2 and o["best_node"][0] == 2
    assert o["accepted_tokens"][0].tolist() == [3, 1, -1, -1]
    assert o["next_token"][0] == 0


@pytest.mark.parametrize("seed", range(6))
def test_accept_matches_path_enumeration(seed):
    """Random trees and logits: the oracle's (accept_len, best_node, tokens)
    equal brute-force enumeration of all root..node paths, given the valid
    bits; valid bits equal a direct argmax check (greedy)."""
    rng = np.random.default_rng(seed)
    K, s, V, B = 5, 3, 6, 4
    t = W.random_tree(200 + seed, 30, K, s)
    ids = np.stack([np.stack([rng.choice(V, s, replace=False) for _ in range(K)])
                    for _ in range(B)]).astype(np.int32)
    L = rng.integers(0, 3, size=(B, t.T, V)).astype(np.float32)  # many ties
    o = oracle.tree_accept(L, ids, t.parent, "f32", "greedy")
    tok = W.path_tokens(t, ids)
    np.testing.assert_array_equal(o["node_tokens"], tok)
    for b in range(B):
        for n in range(1, t.T):
            row = L[b, t.parent[n]]
            am = int(np.flatnonzero(row == row.max())[0])
            assert o["valid"][b, n] == (tok[b, n] == am)
        best, dep = brute.accept_by_paths(t.paths, o["valid"][b])
        assert (o["best_node"][b], o["accept_len"][b]) == (best, dep)
        path = brute.path_nodes(t.paths, best)[1:]
        exp_tokens = [tok[b, m] for m in path] + [-1] * (K - len(path))
        assert o["accepted_tokens"][b].tolist() == exp_tokens
        assert o["next_token"][b] == int(np.argmax(L[b, best]))


def test_accept_bf16_decoding_matches_f32():
    """bf16 logits are decoded exactly: same result as their fp32 values."""
    rng = np.random.default_rng(9)
    t = W.full_product_tree(2, 3)
    ids = np.array([[[1, 2, 3], [4, 5, 6]]], np.int32)
    Lb = W.encode(rng.standard_normal((1, t.T, 10)), W.BF16)
    a = oracle.tree_accept(Lb, ids, t.parent, "bf16", "typical", temperature=0.7)
    b = oracle.tree_accept(W.decode(Lb, W.BF16).astype(np.float32), ids, t.parent, "f32",
                           "typical", temperature=0.7)
    for k in ("valid", "accept_len", "best_node", "accepted_tokens", "next_token"):
        np.testing.assert_array_equal(a[k], b[k])


# ------------------------------------------------------- workload recipe
@pytest.mark.parametrize("name", ["ragged_b16_gqa_typical"])
def test_typical_workload_entropy_spread(name):
    """The typical-mode recipe spreads row entropies over about 0.5-5 nats."""
    wl = W.WORKLOADS[name]
    t = W.workload_tree(wl)
    ids = W.candidate_table(1000 * wl.cid + 12, wl.B, wl.K, wl.s, wl.V)
    tok = W.path_tokens(t, ids)
    logits = W.verify_logits(wl, t, tok)
    o = oracle.tree_accept(logits, ids, t.parent, wl.dtype, "typical", wl.temperature)
    H = o["entropy"][np.isfinite(o["entropy"])]
    assert H.min() < 1.0 and H.max() > 4.0, (H.min(), H.max())
    # decisions are not knife-edge: every child's p/threshold is off 1 by > 1e-3
    r = o["ratio"][:, 1:]
    assert np.all(np.abs(r - 1) > 1e-3)
    assert 0 < o["accept_len"].mean() < wl.K


# ------------------------------------------------------- KV commit (next row f1)
def _kv(B, Hkv, L, T, dh, seed):
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 60000, (B, Hkv, L, dh)).astype(np.uint16)
    vc = rng.integers(0, 60000, (B, Hkv, L, dh)).astype(np.uint16)
    kt = rng.integers(0, 60000, (B, Hkv, T, dh)).astype(np.uint16)
    vt = rng.integers(0, 60000, (B, Hkv, T, dh)).astype(np.uint16)
    return kc, vc, kt, vt


def test_commit_chain_tree_copies_rows_in_order():
    """A chain tree accepted to its tip appends every tree row, in order."""
    kc, vc, kt, vt = _kv(1, 2, 16, 4, 8, 1)
    o = oracle.tree_commit_kv(kc, vc, [5], kt, vt, [3], [-1, 0, 1, 2])
    assert o["committed"].tolist() == [4] and o["prefix_len"].tolist() == [9]
    np.testing.assert_array_equal(o["k_cache"][0, :, 5:9], kt[0])
    np.testing.assert_array_equal(o["v_cache"][0, :, 5:9], vt[0])
    # everything else is untouched
    np.testing.assert_array_equal(o["k_cache"][0, :, :5], kc[0, :, :5])
    np.testing.assert_array_equal(o["k_cache"][0, :, 9:], kc[0, :, 9:])


def test_commit_branching_path_by_hand():
    """Full 2x2 tree (parents -1,0,0,1,1,2,2): node 6's path is 0 -> 2 -> 6."""
    kc, vc, kt, vt = _kv(2, 1, 8, 7, 4, 2)
    parent = [-1, 0, 0, 1, 1, 2, 2]
    o = oracle.tree_commit_kv(kc, vc, [0, 6], kt, vt, [6, 0], parent)
    assert o["committed"].tolist() == [3, 1] and o["prefix_len"].tolist() == [3, 7]
    np.testing.assert_array_equal(o["k_cache"][0, 0, 0:3], kt[0, 0, [0, 2, 6]])
    np.testing.assert_array_equal(o["v_cache"][0, 0, 0:3], vt[0, 0, [0, 2, 6]])
    np.testing.assert_array_equal(o["k_cache"][1, 0, 6], kt[1, 0, 0])   # root only
    np.testing.assert_array_equal(o["k_cache"][1, 0, :6], kc[1, 0, :6])


def test_commit_rejections_leave_the_cache_alone():
    """No room, a length outside [0, Lcap] or a best node outside [0, T):
    nothing is written and the length stays."""
    kc, vc, kt, vt = _kv(4, 1, 8, 3, 4, 3)
    parent = [-1, 0, 1]
    o = oracle.tree_commit_kv(kc, vc, [6, 9, -1, 2], kt, vt, [2, 0, 0, 3], parent)
    assert o["committed"].tolist() == [0, 0, 0, 0]
    assert o["prefix_len"].tolist() == [6, 9, -1, 2]
    np.testing.assert_array_equal(o["k_cache"], kc)
    np.testing.assert_array_equal(o["v_cache"], vc)
    # exactly full: L + path = Lcap fits
    o = oracle.tree_commit_kv(kc, vc, [5, 0, 0, 0], kt, vt, [2, 0, 0, 0], parent)
    assert o["committed"].tolist() == [3, 1, 1, 1] and o["prefix_len"][0] == 8


def test_commit_length_is_depth_plus_one():
    """Rows written = depth(best) + 1 (depth from the C tree oracle)."""
    t = W.pruned_tree(W.WORKLOADS["llama7b_b1"].rates, 3, 64)
    dep = oracle.tree(t.parent, 4, 3)["depth"]
    kc, vc, kt, vt = _kv(1, 1, 64, t.T, 2, 4)
    for best in range(t.T):
        o = oracle.tree_commit_kv(kc, vc, [10], kt, vt, [best], t.parent)
        assert o["committed"][0] == dep[best] + 1


# ------------------------------------------------------- typical variants (next row f3)
def test_loglik_tiebreak_by_hand():
    """Two valid depth-1 children of the root: typical mode keeps the lower
    index, the log-likelihood variant the more probable token."""
    parent = [-1, 0, 0]
    ids = np.array([[[3, 5]]], np.int32)          # node 1 -> token 3, node 2 -> token 5
    logits = np.zeros((1, 3, 8), np.float32)
    logits[0, 0, 3], logits[0, 0, 5] = 2.0, 3.0   # both well above the threshold
    a = oracle.tree_accept(logits, ids, parent, "f32", "typical")
    b = oracle.tree_accept(logits, ids, parent, "f32", "typical_loglik")
    assert a["best_node"][0] == 1 and b["best_node"][0] == 2
    assert a["accept_len"][0] == b["accept_len"][0] == 1
    # the score is ln p of the token under softmax(row): closed form
    p5 = np.exp(3.0) / (np.exp(2.0) + np.exp(3.0) + 6.0)
    assert abs(b["score"][0, 2] - np.log(p5)) < 1e-12
    # equal scores: the lower index wins in both modes
    logits[0, 0, 5] = 2.0
    b = oracle.tree_accept(logits, ids, parent, "f32", "typical_loglik")
    assert b["best_node"][0] == 1


@pytest.mark.parametrize("seed", range(6))
def test_loglik_matches_path_enumeration(seed):
    """Brute force: among the deepest all-valid paths, the one whose summed
    log-softmax probability (scipy's log_softmax) is largest."""
    from scipy.special import log_softmax
    rng = np.random.default_rng(100 + seed)
    t = W.random_tree(seed, 20, 3, 3)
    V, tau = 12, 0.8
    ids = np.stack([rng.permutation(V)[:3] for _ in range(3)])[None].astype(np.int32)
    logits = (rng.standard_normal((1, t.T, V)) * 2).astype(np.float32)
    o = oracle.tree_accept(logits, ids, t.parent, "f32", "typical_loglik", temperature=tau)
    dep = oracle.tree(t.parent, 3, 3)["depth"]
    tok = o["node_tokens"][0]
    lsm = log_softmax(logits[0].astype(np.float64) / tau, axis=-1)
    best, key = 0, (0, 0.0)
    for n in range(1, t.T):
        path = []
        a = n
        while a > 0:
            path.append(a)
            a = t.parent[a]
        if all(o["valid"][0][a] for a in path):
            sc = sum(lsm[t.parent[a], tok[a]] for a in path)
            if (dep[n], sc) > key:
                best, key = n, (dep[n], sc)
    assert o["best_node"][0] == best
    assert o["accept_len"][0] == dep[best]


def test_sample_special_cases():
    V = 10
    x = np.zeros((3, 2, V), np.float32)
    x[0, 1, 7] = 60.0                                  # one-hot in effect
    o = oracle.sample_token(x, [1, 0, 0], [0.99, 0.0, 1 - 1e-12], 1.0, "f32")
    assert o["token"].tolist() == [7, 0, V - 1]        # u = 0 -> first, u -> 1 -> last
    # uniform rows: token = floor(u * V)
    us = np.linspace(0.0, 0.999, 37)
    for uu in us:
        o = oracle.sample_token(np.zeros((1, 1, V), np.float32), [0], [uu], 0.7, "f32")
        assert o["token"][0] == int(np.floor(uu * V + 1e-9))
    # u on a boundary: four equal logits give P(<= t) = (t + 1) / 4 exactly,
    # and the draw is the first t whose P(<= t) exceeds u, so u = k / 4 -> k
    for k in range(4):
        o = oracle.sample_token(np.zeros((1, 1, 4), np.float32), [0], [k / 4], 1.0, "f32")
        assert o["token"][0] == k
    # invalid row or u -> -1
    o = oracle.sample_token(x, [2, 0, -1], [0.5, 1.0, 0.5], 1.0, "f32")
    assert o["token"].tolist() == [-1, -1, -1]


def test_sample_stratified_counts_match_softmax():
    """With the stratified uniforms (k + 1/2) / N every token is drawn
    floor or ceil of N p times (inversion of the distribution function)."""
    rng = np.random.default_rng(3)
    V, N, tau = 9, 2000, 0.6
    row = rng.standard_normal(V).astype(np.float32)
    x = np.broadcast_to(row, (N, 1, V)).copy()
    u = (np.arange(N) + 0.5) / N
    tok = oracle.sample_token(x, np.zeros(N, np.int32), u, tau, "f32")["token"]
    p = np.exp(row / tau - (row / tau).max())
    p /= p.sum()
    cnt = np.bincount(tok, minlength=V)
    assert np.all(np.abs(cnt - N * p) <= 1.0 + 1e-9), (cnt, N * p)


def test_sample_temperature_is_a_logit_scale():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 3, 50)).astype(np.float32)
    u = rng.random(5)
    a = oracle.sample_token(x, [0, 1, 2, 0, 1], u, 0.5, "f32")["token"]
    b = oracle.sample_token((x / np.float32(0.5)).astype(np.float32), [0, 1, 2, 0, 1], u, 1.0,
                            "f32")["token"]
    np.testing.assert_array_equal(a, b)


# ------------------------------------------------------- root token (next row f2)
def test_lm_head_identity_and_planted_rows():
    rng = np.random.default_rng(6)
    d = 16
    h = rng.standard_normal((3, d)).astype(np.float32)
    # identity head: the logits are h itself
    o = oracle.lm_head_argmax(h, np.eye(d, dtype=np.float32), "f32")
    np.testing.assert_array_equal(o["token"], np.argmax(h, axis=1))
    np.testing.assert_allclose(o["logits"], h.astype(np.float64), rtol=0, atol=0)
    # a row equal to 2h dominates (Cauchy-Schwarz against rows of norm <= |h|)
    w = rng.standard_normal((40, d)).astype(np.float32)
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    w *= np.linalg.norm(h[0]) * 0.5
    w[29] = 2 * h[0]
    assert oracle.lm_head_argmax(h[:1], w, "f32")["token"][0] == 29


def test_lm_head_ties_and_bf16_decoding():
    h = np.ones((1, 8), np.float32)
    w = np.zeros((6, 8), np.float32)
    w[2] = w[4] = 1.0 / 8                 # equal logits 1.0 at ids 2 and 4
    assert oracle.lm_head_argmax(h, w, "f32")["token"][0] == 2
    # bf16 bit patterns decode exactly: same as their fp32 values
    rng = np.random.default_rng(7)
    hb = W.encode(rng.standard_normal((2, 32)), W.BF16)
    wb = W.encode(rng.standard_normal((50, 32)), W.BF16)
    a = oracle.lm_head_argmax(hb, wb, "bf16")
    b = oracle.lm_head_argmax(W.decode(hb, W.BF16).astype(np.float32),
                              W.decode(wb, W.BF16).astype(np.float32), "f32")
    np.testing.assert_array_equal(a["token"], b["token"])


# ------------------------------------------------------- multi-layer verify forward (next row f4)
def test_round_to_bf16_matches_torch():
    import torch
    x = np.random.default_rng(1).standard_normal(1000) * 10
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to(x, "bf16"), ref)


def test_rope_closed_forms():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((5, 64))
    k = rng.standard_normal((5, 64))
    np.testing.assert_allclose(oracle.rope(q, np.zeros(5), 1e4), q, atol=1e-15)
    # each (j, j + dh/2) pair keeps its norm
    r = oracle.rope(q, np.arange(5) * 37.0, 1e4)
    np.testing.assert_allclose(r[:, :32] ** 2 + r[:, 32:] ** 2, q[:, :32] ** 2 + q[:, 32:] ** 2,
                               rtol=1e-12)
    # the score depends on the position difference only
    m, n = np.array([40.0, 7.0, 1000.0, 3.0, 0.0]), np.array([3.0, 7.0, 999.0, 30.0, 5.0])
    a = np.sum(oracle.rope(q, m, 1e4) * oracle.rope(k, n, 1e4), axis=1)
    b = np.sum(oracle.rope(q, m - n, 1e4) * k, axis=1)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def test_rmsnorm_unit_rms():
    x = np.random.default_rng(3).standard_normal((4, 256)) * 5
    y = oracle.rmsnorm(x, np.ones(256), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12)


def _fwd_inputs(seed, B, T, d, Hq, Hkv, dh, V, Lcap, N, dtype):
    rng = np.random.default_rng(seed)
    enc = lambda a: oracle.encode(oracle.round_to(a, dtype), dtype)
    layers = [{"g": enc(1 + 0.1 * rng.standard_normal(d)),
               "wq": enc(rng.standard_normal((Hq * dh, d)) / np.sqrt(d)),
               "wk": enc(rng.standard_normal((Hkv * dh, d)) / np.sqrt(d)),
               "wv": enc(rng.standard_normal((Hkv * dh, d)) / np.sqrt(d)),
               "wo": enc(rng.standard_normal((d, Hq * dh)) / np.sqrt(Hq * dh))} for _ in range(N)]
    kc = [enc(rng.standard_normal((B, Hkv, Lcap, dh))) for _ in range(N)]
    vc = [enc(rng.standard_normal((B, Hkv, Lcap, dh))) for _ in range(N)]
    return dict(h0=enc(rng.standard_normal((B, T, d))), layers=layers,
                g_final=enc(np.ones(d)), w_lm=enc(rng.standard_normal((V, d)) / np.sqrt(d)),
                k_caches=kc, v_caches=vc)


def _causal_forward(x, Lb, layers, g_final, w_lm, kc, vc, Hq, Hkv, dh, dtype, b):
    """Plain causal decoding of one sequence: token i at position Lb + i sees
    the cached prefix and tokens 0..i (torch's scaled_dot_product_attention
    with is_causal-style masking)."""
    import torch
    dec = lambda a: oracle.decode(a, dtype)
    h = dec(x)                                       # [n][d]
    n = h.shape[0]
    pos = Lb + np.arange(n, dtype=np.float64)
    G = Hq // Hkv
    for li, lw in enumerate(layers):
        xn = oracle.round_to(oracle.rmsnorm(h, dec(lw["g"]), 1e-6), dtype)
        q = oracle.round_to(oracle.rope((xn @ dec(lw["wq"]).T).reshape(n, Hq, dh).transpose(1, 0, 2),
                                        pos, 1e4), dtype)
        k = oracle.round_to(oracle.rope((xn @ dec(lw["wk"]).T).reshape(n, Hkv, dh).transpose(1, 0, 2),
                                        pos, 1e4), dtype)
        v = oracle.round_to((xn @ dec(lw["wv"]).T).reshape(n, Hkv, dh).transpose(1, 0, 2), dtype)
        K = np.concatenate([dec(kc[li])[b, :, :Lb], k], axis=1)
        Vv = np.concatenate([dec(vc[li])[b, :, :Lb], v], axis=1)
        mask = np.concatenate([np.ones((n, Lb), bool), np.tril(np.ones((n, n), bool))], axis=1)
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(np.repeat(K, G, axis=0)),
            torch.from_numpy(np.repeat(Vv, G, axis=0)), attn_mask=torch.from_numpy(mask)).numpy()
        o = oracle.round_to(o, dtype).transpose(1, 0, 2).reshape(n, Hq * dh)
        h = h + o @ dec(lw["wo"]).T
    xf = oracle.round_to(oracle.rmsnorm(h, dec(g_final), 1e-6), dtype)
    return xf @ dec(w_lm).T


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_chain_tree_is_causal_decoding(dtype):
    B, T, d, Hq, Hkv, dh, V, Lcap, N = 2, 6, 64, 4, 2, 16, 50, 12, 2
    I = _fwd_inputs(11, B, T, d, Hq, Hkv, dh, V, Lcap, N, dtype)
    parent = np.arange(-1, T - 1, dtype=np.int32)
    L = np.array([12, 5], np.int32)
    o = oracle.verify_forward(I["h0"], I["layers"], I["g_final"], I["w_lm"], I["k_caches"],
                              I["v_caches"], L, parent, Hq, Hkv, dh, dtype)
    for b in range(B):
        ref = _causal_forward(I["h0"][b], int(L[b]), I["layers"], I["g_final"], I["w_lm"],
                              I["k_caches"], I["v_caches"], Hq, Hkv, dh, dtype, b)
        np.testing.assert_allclose(o["logits"][b], ref, rtol=1e-9, atol=1e-9)


def test_forward_each_node_is_its_path_decoded():
    """A branching tree: every node's logits equal causal decoding of its
    root -> node path."""
    dtype = "f32"
    B, d, Hq, Hkv, dh, V, Lcap, N = 1, 32, 2, 1, 16, 30, 9, 3
    t = W.full_product_tree(2, 2)                     # 7 nodes
    I = _fwd_inputs(12, B, t.T, d, Hq, Hkv, dh, V, Lcap, N, dtype)
    o = oracle.verify_forward(I["h0"], I["layers"], I["g_final"], I["w_lm"], I["k_caches"],
                              I["v_caches"], [7], t.parent, Hq, Hkv, dh, dtype)
    for n in range(t.T):
        path = []
        a = n
        while a != -1:
            path.append(a)
            a = int(t.parent[a])
        path = path[::-1]
        ref = _causal_forward(I["h0"][0, path], 7, I["layers"], I["g_final"], I["w_lm"],
                              I["k_caches"], I["v_caches"], Hq, Hkv, dh, dtype, 0)
        np.testing.assert_allclose(o["logits"][0, n], ref[-1], rtol=1e-9, atol=1e-9)


def test_forward_without_layers_is_the_lm_head():
    I = _fwd_inputs(13, 1, 3, 32, 2, 2, 16, 20, 4, 0, "f32")
    o = oracle.verify_forward(I["h0"], [], I["g_final"], I["w_lm"], [np.zeros((1, 2, 4, 16), np.float32)],
                              [], [4], [-1, 0, 0], 2, 2, 16, "f32")
    h = oracle.decode(I["h0"], "f32")[0]
    x = oracle.round_to(oracle.rmsnorm(h, 1.0, 1e-6), "f32")      # the one rounding point
    np.testing.assert_allclose(o["logits"][0], x @ oracle.decode(I["w_lm"], "f32").T, rtol=1e-12)


def test_forward_zero_output_projection_keeps_the_residual():
    """Wo = 0: every block adds nothing, so h stays h0 and the logits are the
    LM head on rmsnorm(h0) (catches a dropped or doubled residual)."""
    I = _fwd_inputs(14, 2, 5, 32, 2, 1, 16, 20, 6, 3, "f32")
    for lw in I["layers"]:
        lw["wo"] = np.zeros_like(lw["wo"])
    par = [-1, 0, 0, 1, 2]
    o = oracle.verify_forward(I["h0"], I["layers"], I["g_final"], I["w_lm"], I["k_caches"],
                              I["v_caches"], [3, 6], par, 2, 1, 16, "f32")
    z = oracle.verify_forward(I["h0"], [], I["g_final"], I["w_lm"], I["k_caches"], [], [3, 6],
                              par, 2, 1, 16, "f32")
    np.testing.assert_array_equal(o["hidden"], oracle.decode(I["h0"], "f32"))
    np.testing.assert_allclose(o["logits"], z["logits"], rtol=1e-12)


def test_forward_uniform_attention_by_hand():
    """Wq = 0 makes every score 0, so a node's attention output is the mean
    of the visible values: the L_b cached rows and its ancestors-or-self.
    With Wv = I, the values of the tree are x itself; Wo is a permutation
    (y[i] = o[pi(i)] in the [out][in] layout), which pins its orientation."""
    d = dh = 16
    rng = np.random.default_rng(15)
    h0 = rng.standard_normal((1, 4, d)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    pi = np.roll(np.arange(d), 3)                       # not an involution
    wo = np.zeros((d, d), np.float32)
    wo[np.arange(d), pi] = 1.0
    layer = {"g": g, "wq": np.zeros((d, d), np.float32), "wk": rng.standard_normal((d, d)).astype(np.float32),
             "wv": np.eye(d, dtype=np.float32), "wo": wo}
    L, Lcap = 3, 5
    kc = rng.standard_normal((1, 1, Lcap, dh)).astype(np.float32)
    vc = rng.standard_normal((1, 1, Lcap, dh)).astype(np.float32)
    par = [-1, 0, 1, 0]
    o = oracle.verify_forward(h0, [layer], np.ones(d, np.float32), np.eye(d, dtype=np.float32),
                              [kc], [vc], [L], par, 1, 1, dh, "f32")
    h = h0[0].astype(np.float64)
    x = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + 1e-6) * g
    x = x.astype(np.float32).astype(np.float64)         # the fp32 rounding point
    paths = {0: [0], 1: [0, 1], 2: [0, 1, 2], 3: [0, 3]}
    for n in range(4):
        att = (vc[0, 0, :L].astype(np.float64).sum(0) + x[paths[n]].sum(0)) / (L + len(paths[n]))
        att = att.astype(np.float32).astype(np.float64)
        np.testing.assert_allclose(o["hidden"][0, n], h[n] + att[pi], rtol=1e-12, atol=1e-12)
