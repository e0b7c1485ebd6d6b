"""GPU parity: tree_commit_kv against the CPU oracle (a copy: bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from medusa_tree_verification_amd import workloads as W
from tests.util import to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.cpu().numpy()


def _run(kc, vc, L, kt, vt, best, parent):
    from medusa_tree_verification_amd import binding as mv
    d = {k: to_dev(v) for k, v in dict(kc=kc, vc=vc, kt=kt, vt=vt).items()}
    Ld = to_dev(np.asarray(L, np.int32))
    com = torch.full((len(L),), -5, dtype=torch.int32, device="cuda")
    mv.tree_commit_kv(d["kc"], d["vc"], Ld, d["kt"], d["vt"], to_dev(np.asarray(best, np.int32)),
                      parent, committed=com)
    torch.cuda.synchronize()
    return {"k_cache": _bits(d["kc"]), "v_cache": _bits(d["vc"]), "prefix_len": Ld.cpu().numpy(),
            "committed": com.cpu().numpy()}


def _rand(rng, shape, dtype):
    if dtype == "bf16":
        return rng.integers(0, 1 << 16, shape).astype(np.uint16)
    return rng.standard_normal(shape).astype(np.float32)


def _check(g, r):
    for k in ("k_cache", "v_cache", "prefix_len", "committed"):
        np.testing.assert_array_equal(g[k], r[k], err_msg=k)


@pytest.mark.parametrize("dtype,dh", [("bf16", 128), ("bf16", 64), ("f32", 64), ("bf16", 8)])
def test_commit_random(dtype, dh):
    rng = np.random.default_rng(dh + (dtype == "f32"))
    B, Hkv, Lcap = 7, 3, 40
    t = W.random_tree(11, 37, 5, 3)
    kc, vc = _rand(rng, (B, Hkv, Lcap, dh), dtype), _rand(rng, (B, Hkv, Lcap, dh), dtype)
    kt, vt = _rand(rng, (B, Hkv, t.T, dh), dtype), _rand(rng, (B, Hkv, t.T, dh), dtype)
    dep = oracle.tree(t.parent, 64, 64)["depth"]
    deep = int(np.argmax(dep))                          # path of dep + 1 rows fills to Lcap
    # room, exactly full, no room, empty prefix, bad length, bad best node, root only
    L = [10, Lcap - int(dep[deep]) - 1, Lcap - 1, 0, Lcap + 1, 3, 39]
    best = [t.T - 1, deep, t.T - 2, 17, 5, t.T, 0]
    _check(_run(kc, vc, L, kt, vt, best, t.parent),
           oracle.tree_commit_kv(kc, vc, L, kt, vt, best, t.parent))


def test_commit_twice_appends_twice():
    rng = np.random.default_rng(5)
    t = W.full_product_tree(3, 2)
    kc, vc = _rand(rng, (2, 2, 32, 64), "bf16"), _rand(rng, (2, 2, 32, 64), "bf16")
    kt, vt = _rand(rng, (2, 2, t.T, 64), "bf16"), _rand(rng, (2, 2, t.T, 64), "bf16")
    from medusa_tree_verification_amd import binding as mv
    d = [to_dev(x) for x in (kc, vc, kt, vt)]
    Ld = to_dev(np.array([3, 20], np.int32))
    for best in ([14, 1], [7, 0]):
        mv.tree_commit_kv(d[0], d[1], Ld, d[2], d[3], to_dev(np.array(best, np.int32)), t.parent)
    torch.cuda.synchronize()
    r = oracle.tree_commit_kv(kc, vc, [3, 20], kt, vt, [14, 1], t.parent)
    r = oracle.tree_commit_kv(r["k_cache"], r["v_cache"], r["prefix_len"], kt, vt, [7, 0], t.parent)
    np.testing.assert_array_equal(_bits(d[0]), r["k_cache"])
    np.testing.assert_array_equal(_bits(d[1]), r["v_cache"])
    np.testing.assert_array_equal(Ld.cpu().numpy(), r["prefix_len"])


@pytest.mark.parametrize("name", ["ragged_b16_gqa_typical", "large_vocab_typical"])
def test_commit_workload_shapes(name):
    """Full workload shapes, cache capacity grown by T rows; best nodes of
    every depth."""
    wl = W.WORKLOADS[name]
    t = W.workload_tree(wl)
    ax = W.attention_inputs(wl)
    rng = np.random.default_rng(wl.cid)
    Lcap = wl.Lcap + t.T
    kc = np.zeros((wl.B, wl.Hkv, Lcap, wl.dh), np.uint16)
    vc = np.zeros_like(kc)
    kc[:, :, :wl.Lcap] = ax["k_cache"]
    vc[:, :, :wl.Lcap] = ax["v_cache"]
    best = rng.integers(0, t.T, wl.B)
    _check(_run(kc, vc, ax["prefix_len"], ax["k_tree"], ax["v_tree"], best, t.parent),
           oracle.tree_commit_kv(kc, vc, ax["prefix_len"], ax["k_tree"], ax["v_tree"], best,
                                 t.parent))
