"""GPU parity: medusa_heads_topk against the CPU oracle (through the C ABI)."""
import numpy as np
import pytest

import oracle
from medusa_tree_verification_amd import workloads as W
from tests.util import from_dev, normwise, to_dev, topk_check

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _run(hx, s, dtype, **kw):
    from medusa_tree_verification_amd import binding as mv
    out = mv.medusa_heads_topk(to_dev(hx["hidden"]), to_dev(hx["w1"]), to_dev(hx["w2"]), s,
                               want_logits=True, **kw)
    return {k: v.cpu().numpy() for k, v in out.items()}


def _compare(out, ref, s, dtype):
    err = normwise(out["logits"], ref["logits"], axes=2)
    assert err.max() < TOL[dtype], err.max()
    amb = topk_check(out["topk_ids"], ref["logits"], ref["topk_ids"], s, out["logits"])
    # values reported with the ids are the logits of those ids
    B, K, _ = ref["logits"].shape
    vals_ref = np.take_along_axis(ref["logits"], out["topk_ids"].astype(np.int64), axis=2)
    assert normwise(out["topk_vals"], vals_ref, axes=(1, 2)).max() < TOL[dtype]
    return amb


def _random_heads(seed, B, K, d, V, dtype, wstd=0.05):
    return {"hidden": W.normal_tensor(seed + 1, (B, d), 1.0, dtype),
            "w1": W.normal_tensor(seed + 2, (K, d, d), wstd, dtype),
            "w2": W.normal_tensor(seed + 3, (K, V, d), wstd, dtype)}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,K,d,V,s", [
    (1, 1, 128, 16, 1),        # one tile
    (1, 3, 256, 1000, 2),      # ragged last tile
    (3, 2, 384, 777, 8),       # s = 8, odd batch
    (2, 3, 256, 2000, 4),      # s = 4: every slot of the short lists
    (5, 2, 256, 1500, 5),      # s = 5: the long lists
    (16, 5, 256, 4099, 3),     # full batch tile, tiles spanning head boundaries
    (7, 4, 128, 70000, 3),     # many tiles per workgroup
])
def test_heads_random_shapes(dtype, B, K, d, V, s):
    hx = _random_heads(hash((B, K, d, V, s)) % 10000 * 10, B, K, d, V, dtype)
    out = _run(hx, s, dtype)
    ref = oracle.heads_topk(hx["hidden"], hx["w1"], hx["w2"], s, dtype)
    amb = _compare(out, ref, s, dtype)
    assert amb <= max(1, B * K // 20)


def test_heads_four_tile_stage1_partial_batch():
    # K * d / 64 = 256 tile groups and B >= 4: stage 1 gives each workgroup
    # four tiles; 6 of the 16 MFMA columns hold sequences
    B, K, d, V, s = 6, 4, 4096, 300, 3
    hx = _random_heads(4242, B, K, d, V, "bf16")
    out = _run(hx, s, "bf16")
    ref = oracle.heads_topk(hx["hidden"], hx["w1"], hx["w2"], s, "bf16")
    amb = _compare(out, ref, s, "bf16")
    assert amb <= 1


def test_heads_four_tile_stage1_f32():
    B, K, d, V, s = 4, 4, 4096, 200, 3
    hx = _random_heads(4343, B, K, d, V, "f32")
    out = _run(hx, s, "f32")
    ref = oracle.heads_topk(hx["hidden"], hx["w1"], hx["w2"], s, "f32")
    amb = _compare(out, ref, s, "f32")
    assert amb <= 1


def test_heads_five_tile_stage1_across_heads():
    # K = 5 heads of 4096 rows: stage 1 runs 256 workgroups of five tiles,
    # and the groups that straddle a head boundary write into two heads
    B, K, d, V, s = 5, 5, 4096, 300, 3
    hx = _random_heads(5151, B, K, d, V, "bf16")
    out = _run(hx, s, "bf16")
    ref = oracle.heads_topk(hx["hidden"], hx["w1"], hx["w2"], s, "bf16")
    amb = _compare(out, ref, s, "bf16")
    assert amb <= 1


def test_heads_exact_small_integers():
    """Values on a coarse binary grid make every fp32 sum exact: logits must be
    bit-identical to the oracle's."""
    rng = np.random.default_rng(5)
    B, K, d, V, s = 4, 2, 128, 300, 3
    hx = {"hidden": rng.integers(-4, 5, size=(B, d)).astype(np.float32),
          "w1": np.zeros((K, d, d), np.float32),
          "w2": (rng.integers(-1, 2, size=(K, V, d)) / 16.0).astype(np.float32)}
    out = _run(hx, s, "f32")
    ref = oracle.heads_topk(hx["hidden"], hx["w1"], hx["w2"], s, "f32")
    np.testing.assert_array_equal(out["logits"].astype(np.float64), ref["logits"])
    np.testing.assert_array_equal(out["topk_ids"], ref["topk_ids"])  # many exact ties


@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_heads_workloads(name):
    wl = W.WORKLOADS[name]
    hx = W.heads_inputs(wl)
    out = _run(hx, wl.s, wl.dtype)
    ref = oracle.heads_topk(hx["hidden"], hx["w1"], hx["w2"], wl.s, wl.dtype)
    amb = _compare(out, ref, wl.s, wl.dtype)
    print(f"{name}: near-tie top-s rows {amb} of {wl.B * wl.K}")
    assert amb <= 1


def test_heads_stages_equal_fused_call_and_repeat_bit_identical():
    from medusa_tree_verification_amd import binding as mv
    import torch
    wl = W.WORKLOADS["llama7b_b1"]
    hx = _random_heads(777, 5, 4, 512, 5000, "bf16")
    h, w1, w2 = (to_dev(hx[k]) for k in ("hidden", "w1", "w2"))
    B, K, d, V, s = 5, 4, 512, 5000, 3
    a = mv.medusa_heads_topk(h, w1, w2, s, want_logits=True)
    ws = mv.workspace(mv.lib.medusa_heads_topk_workspace_bytes(B, K, d, V, s, mv.BF16), h.device)
    ids = torch.empty((B, K, s), dtype=torch.int32, device=h.device)
    vals = torch.empty((B, K, s), dtype=torch.float32, device=h.device)
    lg = torch.empty((B, K, V), dtype=torch.float32, device=h.device)
    for _ in range(3):
        mv.medusa_heads_stage1(h, w1, B, K, d, V, s, ws)
        mv.medusa_heads_stage2(w2, B, K, d, V, s, ids, ws, topk_vals=vals, logits=lg)
        torch.cuda.synchronize()
        assert torch.equal(ids, a["topk_ids"]) and torch.equal(vals, a["topk_vals"])
        assert torch.equal(lg, a["logits"])
    # the stream and the merge as separate calls give the same bits
    ids.fill_(-1)
    vals.zero_()
    mv.medusa_heads_stage1(h, w1, B, K, d, V, s, ws)
    mv.medusa_heads_stage2_stream(w2, B, K, d, V, s, ws)
    mv.medusa_heads_stage2_merge(B, K, d, V, s, mv.BF16, ids, ws, topk_vals=vals)
    torch.cuda.synchronize()
    assert torch.equal(ids, a["topk_ids"]) and torch.equal(vals, a["topk_vals"])
    del wl


# ---------------------------------------------------------------- root token
def _root_run(hx, s):
    from medusa_tree_verification_amd import binding as mv
    out = mv.medusa_heads_topk_root(to_dev(hx["hidden"]), to_dev(hx["w1"]), to_dev(hx["w2"]),
                                    to_dev(hx["w_lm"]), s)
    return {k: v.cpu().numpy() for k, v in out.items()}


def _root_check(out, hx, dtype):
    """The GPU's root must be the oracle's argmax unless the oracle's top two
    logits are within the GPU's own logit error (then it must be within that
    error of the maximum).  Returns the number of such near-tie rows."""
    ref = oracle.lm_head_argmax(hx["hidden"], hx["w_lm"], dtype)
    lg = ref["logits"]
    near = 0
    for b in range(lg.shape[0]):
        t = int(out["root_token"][b])
        band = 4 * max(abs(float(out["root_val"][b]) - lg[b, t]), 1e-6 * np.abs(lg[b]).max())
        top2 = np.sort(lg[b])[-2:] if lg.shape[1] > 1 else np.array([lg[b, 0], -np.inf])
        assert lg[b, t] >= top2[-1] - band, (b, t, lg[b, t], top2)
        if top2[-1] - top2[-2] > band:
            assert t == ref["token"][b]
        else:
            near += 1
    return near


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,K,d,V,s", [(1, 1, 128, 16, 1), (3, 2, 384, 777, 8),
                                       (16, 5, 256, 4099, 3), (7, 4, 128, 70000, 3)])
def test_heads_root_random(dtype, B, K, d, V, s):
    seed = hash((B, K, d, V, s, 7)) % 10000 * 10
    hx = _random_heads(seed, B, K, d, V, dtype)
    hx["w_lm"] = W.normal_tensor(seed + 4, (V, d), 0.05, dtype)
    out = _root_run(hx, s)
    # the Medusa heads' results are those of the plain call (the extra head
    # moves the work split, hence the order of the k-sums: values agree to
    # rounding, ids except where two candidates are that close)
    plain = _run(hx, s, dtype)
    np.testing.assert_allclose(out["topk_vals"], plain["topk_vals"], rtol=1e-5, atol=1e-6)
    diff = out["topk_ids"] != plain["topk_ids"]
    np.testing.assert_allclose(out["topk_vals"][diff], plain["topk_vals"][diff], rtol=1e-5)
    assert _root_check(out, hx, dtype) <= max(1, B // 8)


def test_heads_root_workload_shape():
    """Llama-7B shapes (d 4096, V 32000, bf16) with a planted root per row."""
    wl = W.WORKLOADS["ragged_b16_gqa_typical"]
    hx = W.heads_inputs(wl)
    w_lm = W.normal_tensor(1000 * wl.cid + 20, (wl.V, wl.d), 0.02, wl.dtype)
    h = W.decode(hx["hidden"], wl.dtype)
    rng = np.random.default_rng(21)
    plant = rng.choice(wl.V, wl.B, replace=False)
    for b in range(wl.B):
        w_lm[plant[b]] = W.encode(h[b] / np.linalg.norm(h[b]) * 0.5, wl.dtype)
    hx["w_lm"] = w_lm
    out = _root_run(hx, wl.s)
    assert _root_check(out, hx, wl.dtype) == 0
    np.testing.assert_array_equal(out["root_token"], plant)
