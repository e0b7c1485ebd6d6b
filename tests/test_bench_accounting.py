"""CPU: the bench's roofline accounting (algorithmic bytes and FLOPs) against
counts made independently: closed forms for the weight streams, and a brute
count of the visible (query, key) pairs of the tree attention."""
import numpy as np

import bench
from medusa_tree_verification_amd import workloads as W


def test_heads_bytes_closed_forms():
    wl = W.WORKLOADS["llama7b_b1"]
    t = W.workload_tree(wl)
    n_int = len(set(int(x) for x in t.parent[1:]))
    nb = bench.algorithmic_bytes(wl, W.prefix_lengths(wl), n_int)
    # W2 of 4 heads x 32000 x 4096 bf16, plus z (1 x 4 x 4096 bf16)
    assert nb["heads_stage2"] == 4 * 32000 * 4096 * 2 + 4 * 4096 * 2 == 1_048_608_768
    # W1 of 4 heads x 4096 x 4096, h in, z out
    assert nb["heads_stage1"] == 4 * 4096 * 4096 * 2 + 4096 * 2 + 4 * 4096 * 2
    # the merge writes ids and values: B x K x s x 8 bytes
    assert nb["heads_merge"] == 1 * 4 * 3 * 8
    # acceptance reads every internal row and the best row once
    assert nb["tree_accept"] == 1 * (n_int + 1) * 32000 * 2


def _visible_pairs(tree, prefix_len, Hq):
    """Brute force: every (sequence, query head, node) sees its prefix and
    the nodes on its root path (itself included)."""
    n = 0
    for L in prefix_len:
        for node in range(tree.T):
            anc, a = 0, node
            while True:
                anc += 1
                if a == 0:
                    break
                a = int(tree.parent[a])
            n += Hq * (int(L) + anc)
    return n


def test_attention_flops_count_visible_pairs():
    for name in ("tiny_fp32", "ragged_b16_gqa_typical", "large_vocab_typical"):
        wl = W.WORKLOADS[name]
        t = W.workload_tree(wl)
        L = np.minimum(W.prefix_lengths(wl), wl.Lcap)
        # q.k and p.v: 2 flops per multiply-add, dh of each per visible pair
        assert bench.attention_flops(wl, L, t) == 4 * wl.dh * _visible_pairs(t, L, wl.Hq), name


def test_attention_bytes_read_kv_once():
    wl = W.WORKLOADS["ragged_b16_gqa_typical"]
    t = W.workload_tree(wl)
    L = W.prefix_lengths(wl)
    n_int = len(set(int(x) for x in t.parent[1:]))
    nb = bench.algorithmic_bytes(wl, L, n_int)["tree_attention"]
    w = 2
    kv_prefix = 2 * wl.Hkv * int(np.minimum(L, wl.Lcap).sum()) * wl.dh * w
    kv_tree = 2 * wl.B * wl.Hkv * wl.T * wl.dh * w
    q_and_out = 2 * wl.B * wl.Hq * wl.T * wl.dh * w
    assert nb == kv_prefix + kv_tree + q_and_out
