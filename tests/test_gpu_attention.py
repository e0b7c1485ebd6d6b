"""GPU parity: tree_attention against the CPU oracle (through the C ABI)."""
import math

import numpy as np
import pytest

import oracle
from medusa_tree_verification_amd import workloads as W
from tests.util import Canaries, from_dev, normwise, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _inputs(seed, B, Hq, Hkv, T, dh, Lcap, L, dtype):
    f = lambda k, *sh: W.normal_tensor(seed + k, sh, 1.0, dtype)
    return dict(q=f(1, B, Hq, T, dh), k_cache=f(2, B, Hkv, Lcap, dh), v_cache=f(3, B, Hkv, Lcap, dh),
                k_tree=f(4, B, Hkv, T, dh), v_tree=f(5, B, Hkv, T, dh),
                prefix_len=np.asarray(L, np.int32))


def _gpu(x, parent, scale, want_mask=False):
    import torch
    from medusa_tree_verification_amd import binding as mv
    d = {k: to_dev(v) for k, v in x.items()}
    T = d["q"].shape[2]
    cz = Canaries()
    out = cz.like(d["q"])
    mask = cz.empty((T, (T + 63) // 64), torch.int64) if want_mask else None
    mv.tree_attention(d["q"], d["k_cache"], d["v_cache"], d["prefix_len"], d["k_tree"],
                      d["v_tree"], parent, scale, out=out, mask_out=mask)
    cz.check()
    if want_mask:
        return from_dev(out), mask.cpu().numpy().view(np.uint64)
    return from_dev(out)


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


@pytest.mark.parametrize("G,dtype", [(2, "bf16"), (4, "bf16"), (4, "f32")])
def test_attention_grid_over_several_rounds(G, dtype):
    # more (sequence, kv head, m-tile) blocks than CUs: 23 sequences x 13 kv
    # heads = 299 blocks, not a multiple of the eight XCDs, so the block
    # remap's uneven ranges and a second round of workgroups both occur;
    # prefixes 0..600 (G = 4, bf16: the pipelined kernel)
    t = W.random_tree(70 + G, 64, 4, 3)
    B, Hkv, dh, Lcap = 23, 13, 128, 600
    L = [(37 * b) % 601 for b in range(B)]
    x = _inputs(600 + G, B, G * Hkv, Hkv, t.T, dh, Lcap, L, dtype)
    _check(x, t.parent, 1 / math.sqrt(dh), dtype)


def test_attention_long_prefix_many_splits():
    t = TREES["full121"]
    B, Hq, Hkv, dh, Lcap = 1, 4, 1, 128, 20000
    x = _inputs(400, B, Hq, Hkv, t.T, dh, Lcap, [19999], "bf16")
    _check(x, t.parent, 1 / math.sqrt(dh), "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_reference_moves(dtype):
    # Scores (log2 units) that step up by 9 per 32-key block over the first
    # six blocks and then stay level: every step lifts the block maximum past
    # the running reference + 8, so the kernels move their reference five
    # times while the next block's q.k products are partly summed, and the
    # blocks after the last move carry nearly all of the softmax weight, so a
    # wrong correction of that partial sum would show in the output.  G * T =
    # 256 rows per kv head (bf16: the pipelined kernel).
    t = W.random_tree(91, 64, 4, 3)
    B, Hkv, G, dh, Lcap = 2, 2, 4, 128, 700
    L = [700, 389]
    Hq, T = G * Hkv, t.T
    scale = 1 / math.sqrt(dh)
    c = scale * math.log2(math.e)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([4242])))
    u = rng.standard_normal(dh).astype(np.float32)
    q = u + 0.1 * rng.standard_normal((B, Hq, T, dh)).astype(np.float32)
    step = 9.0 * np.minimum(np.arange(Lcap) // 32, 5).astype(np.float32)
    k = 0.3 * rng.standard_normal((B, Hkv, Lcap, dh)).astype(np.float32)
    k += (step / (c * float(u @ u)))[None, None, :, None] * u
    conv = (lambda a: W.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    x = dict(q=conv(q), k_cache=conv(k),
             v_cache=conv(rng.standard_normal((B, Hkv, Lcap, dh)).astype(np.float32)),
             k_tree=conv(rng.standard_normal((B, Hkv, T, dh)).astype(np.float32)),
             v_tree=conv(rng.standard_normal((B, Hkv, T, dh)).astype(np.float32)),
             prefix_len=np.asarray(L, np.int32))
    _check(x, t.parent, scale, dtype)


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


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_attention_workloads(name):
    """Every output row of the workload against the oracle."""
    wl = W.WORKLOADS[name]
    t = W.workload_tree(wl)
    x = W.attention_inputs(wl)
    _, _, err = _check(x, t.parent, wl.scale, wl.dtype)
    print(f"{name}: normwise err {err:.3g} over all {wl.B * wl.Hq * wl.T} rows")


@pytest.mark.parametrize("name,dtype", [("ragged_b16_gqa_typical", "bf16"),
                                        ("long_ctx_32k", "bf16"),
                                        ("large_vocab_typical", "bf16"),
                                        ("large_vocab_typical", "f32")])
def test_attention_repeat_bit_identical(name, dtype):
    """The same call three more times gives the same bits (no race in the
    staging ring, the LDS double buffer or the split merge)."""
    wl = W.WORKLOADS[name]
    t = W.workload_tree(wl)
    x = W.attention_inputs(wl)
    if dtype != wl.dtype:
        x = {k: (W.encode(W.decode(v, wl.dtype), dtype) if v.dtype == np.uint16 else v)
             for k, v in x.items()}
    a = _gpu(x, t.parent, wl.scale)
    for _ in range(3):
        np.testing.assert_array_equal(_gpu(x, t.parent, wl.scale), a)
