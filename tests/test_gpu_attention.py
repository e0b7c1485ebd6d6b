"""GPU parity: tree_attention against the CPU oracle (through the C ABI)."""
import math

import numpy as np
import pytest

import oracle
from medusa_tree_verification_amd import workloads as W
from tests.util import from_dev, normwise, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _inputs(seed, B, Hq, Hkv, T, dh, Lcap, L, dtype):
    f = lambda k, *sh: W.normal_tensor(seed + k, sh, 1.0, dtype)
    return dict(q=f(1, B, Hq, T, dh), k_cache=f(2, B, Hkv, Lcap, dh), v_cache=f(3, B, Hkv, Lcap, dh),
                k_tree=f(4, B, Hkv, T, dh), v_tree=f(5, B, Hkv, T, dh),
                prefix_len=np.asarray(L, np.int32))


def _gpu(x, parent, scale, want_mask=False):
    from medusa_tree_verification_amd import binding as mv
    d = {k: to_dev(v) for k, v in x.items()}
    r = mv.tree_attention(d["q"], d["k_cache"], d["v_cache"], d["prefix_len"], d["k_tree"],
                          d["v_tree"], parent, scale, want_mask=want_mask)
    if want_mask:
        return from_dev(r[0]), r[1].cpu().numpy().view(np.uint64)
    return from_dev(r)


def _check(x, tree_parent, scale, dtype, rows=None, want_mask=False):
    g = _gpu(x, tree_parent, scale, want_mask)
    mask = None
    if want_mask:
        g, mask = g
    if rows is None:
        ref = oracle.tree_attention(**x, parent=tree_parent, scale=scale, dtype=dtype)
        err = normwise(g, ref, axes=(2, 3))
    else:
        ref = oracle.tree_attention(**x, parent=tree_parent, scale=scale, dtype=dtype, rows=rows)
        gs = g[rows[:, 0], rows[:, 1], rows[:, 2]]
        err = normwise(gs, ref, axes=1)
    assert np.isfinite(g).all()
    assert err.max() < TOL[dtype], err.max()
    return g, mask, err.max()


TREES = {
    "root": W.tree_from_paths([()]),
    "pair": W.full_product_tree(1, 1),
    "full2x3": W.full_product_tree(3, 2),
    "pruned64": W.pruned_tree(W.WORKLOADS["llama7b_b1"].rates, 3, 64),
    "rand65": W.random_tree(31, 65, 6, 4),
    "full121": W.full_product_tree(4, 3),
    "rand128": W.random_tree(32, 128, 7, 4),
    "pruned256": W.pruned_tree(W.WORKLOADS["large_vocab_typical"].rates, 3, 256),
    "chain9": W.chain_tree(8),
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tree", list(TREES))
def test_attention_trees(dtype, tree):
    t = TREES[tree]
    B, Hq, Hkv, dh, Lcap = 2, 4, 2, 64, 200
    L = [200, 37]
    x = _inputs(100, B, Hq, Hkv, t.T, dh, Lcap, L, dtype)
    _, mask, _ = _check(x, t.parent, 1 / math.sqrt(dh), dtype, want_mask=True)
    ref = oracle.tree(t.parent, t.T, t.T)["mask"]
    np.testing.assert_array_equal(mask, ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [[0, 0], [1, 64], [63, 65], [127, 129], [300, 1000]])
def test_attention_ragged_prefix(dtype, L):
    t = TREES["full2x3"]
    B, Hq, Hkv, dh, Lcap = 2, 8, 2, 128, 1000
    x = _inputs(200, B, Hq, Hkv, t.T, dh, Lcap, L, dtype)
    _check(x, t.parent, 0.09, dtype)


@pytest.mark.parametrize("G,T", [(1, 15), (4, 64), (8, 33), (2, 256), (16, 40)])
def test_attention_gqa_groups(G, T):
    t = W.random_tree(40 + T, T, 8, 3)
    B, Hkv, dh, Lcap = 2, 2, 128, 3000
    x = _inputs(300, B, G * Hkv, Hkv, T, dh, Lcap, [3000, 1234], "bf16")
    _check(x, t.parent, 1 / math.sqrt(dh), "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8])
def test_attention_row_wave_counts(G, dtype):
    # G * 30 query rows per kv head: 1 .. 8 row waves of 32, i.e. every
    # split of the eight waves between row owners (one or two per row tile)
    # and waves that only stage K/V; ragged prefixes over several splits
    t = W.random_tree(60 + G, 30, 4, 3)
    B, Hkv, dh, Lcap = 2, 2, 128, 700
    x = _inputs(350 + G, B, G * Hkv, Hkv, t.T, dh, Lcap, [700, 389], dtype)
    _check(x, t.parent, 1 / math.sqrt(dh), dtype)


def test_attention_long_prefix_many_splits():
    t = TREES["full121"]
    B, Hq, Hkv, dh, Lcap = 1, 4, 1, 128, 20000
    x = _inputs(400, B, Hq, Hkv, t.T, dh, Lcap, [19999], "bf16")
    rows = np.array([[0, h, n] for h in range(Hq) for n in (0, 1, 5, 40, 120)], np.int32)
    _check(x, t.parent, 1 / math.sqrt(dh), "bf16", rows=rows)


def test_attention_prefix_out_of_range_is_clamped_and_flagged():
    from medusa_tree_verification_amd import binding as mv
    import torch
    t = TREES["full2x3"]
    B, Hq, Hkv, dh, Lcap = 2, 2, 2, 64, 100
    x = _inputs(500, B, Hq, Hkv, t.T, dh, Lcap, [150, 50], "f32")
    d = {k: to_dev(v) for k, v in x.items()}
    ws = mv.workspace(mv.lib.tree_attention_workspace_bytes(B, Hq, Hkv, Lcap, dh, t.T, mv.F32),
                      d["q"].device)
    out = mv.tree_attention(d["q"], d["k_cache"], d["v_cache"], d["prefix_len"], d["k_tree"],
                            d["v_tree"], t.parent, 0.125, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) != 0
    ref = oracle.tree_attention(**x, parent=t.parent, scale=0.125, dtype="f32")  # clamps too
    assert normwise(from_dev(out), ref, axes=(2, 3)).max() < 1e-5
    d["prefix_len"].copy_(torch.tensor([100, 50], dtype=torch.int32))
    mv.tree_attention(d["q"], d["k_cache"], d["v_cache"], d["prefix_len"], d["k_tree"],
                      d["v_tree"], t.parent, 0.125, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0


def _sample_rows(wl, n, seed):
    rng = np.random.default_rng(seed)
    rows = np.stack([rng.integers(0, wl.B, n), rng.integers(0, wl.Hq, n),
                     rng.integers(0, wl.T, n)], axis=1).astype(np.int32)
    # always include the root and the last node of the first and last sequence
    extra = np.array([[0, 0, 0], [wl.B - 1, wl.Hq - 1, wl.T - 1], [0, wl.Hq - 1, wl.T - 1]],
                     np.int32)
    return np.concatenate([extra, rows])


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_attention_workloads(name):
    wl = W.WORKLOADS[name]
    t = W.workload_tree(wl)
    x = W.attention_inputs(wl)
    small = wl.B * wl.Hq * wl.T * (int(x["prefix_len"].sum()) + wl.T) * wl.dh < 3e9
    rows = None if small else _sample_rows(wl, 384, wl.cid)
    _, _, err = _check(x, t.parent, wl.scale, wl.dtype, rows=rows)
    print(f"{name}: normwise err {err:.3g} ({'all rows' if rows is None else f'{len(rows)} rows'})")


def test_attention_repeat_bit_identical():
    wl = W.WORKLOADS["ragged_b16_gqa_typical"]
    t = W.workload_tree(wl)
    x = W.attention_inputs(wl)
    a = _gpu(x, t.parent, wl.scale)
    for _ in range(3):
        np.testing.assert_array_equal(_gpu(x, t.parent, wl.scale), a)
