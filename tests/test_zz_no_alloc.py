"""GPU: medusa_heads_topk_noalloc (static scratch, no workspace) gives the
same bits as medusa_heads_topk (caller workspace), on two calls in a row, the
second with a smaller problem, so that the first call's scratch contents are
still there when the second runs."""
import numpy as np
import pytest

from medusa_tree_verification_amd import workloads as W
from tests.util import Canaries, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, B, K, d, V, dtype):
    return {"hidden": W.normal_tensor(seed + 1, (B, d), 1.0, dtype),
            "w1": W.normal_tensor(seed + 2, (K, d, d), 0.02, dtype),
            "w2": W.normal_tensor(seed + 3, (K, V, d), 0.02, dtype)}


def _outputs(cz, B, K, V, s):
    import torch
    return {"topk_ids": cz.empty((B, K, s), torch.int32),
            "topk_vals": cz.empty((B, K, s), torch.float32),
            "logits": cz.empty((B, K, V), torch.float32)}


def test_noalloc_matches_workspace_call_twice_shrinking():
    import torch
    from medusa_tree_verification_amd import binding as mv
    cases = [(8, 5, 4096, 32000, 3, "bf16"),      # larger first
             (3, 2, 1024, 5000, 4, "f32")]        # then smaller, other dtype and s
    for i, (B, K, d, V, s, dt) in enumerate(cases):
        x = _inputs(9100 + 10 * i, B, K, d, V, dt)
        h, w1, w2 = (to_dev(x[k]) for k in ("hidden", "w1", "w2"))
        cz = Canaries()
        ref = mv.medusa_heads_topk(h, w1, w2, s, out=_outputs(cz, B, K, V, s))
        got = mv.medusa_heads_topk_noalloc(h, w1, w2, s, out=_outputs(cz, B, K, V, s))
        cz.check()
        for k in ("topk_ids", "topk_vals", "logits"):
            assert torch.equal(got[k], ref[k]), (i, k)
        print(f"call {i}: B={B} K={K} d={d} V={V} s={s} {dt}: identical to medusa_heads_topk "
              f"(ids {got['topk_ids'][0, 0].tolist()})", flush=True)


def test_noalloc_rejects_oversized_problem_without_touching_outputs():
    import torch
    from medusa_tree_verification_amd import binding as mv
    B, K, d, V, s = 16, 16, 16384, 1000, 3
    # tiny placeholder inputs: the size check fails before any pointer is used
    h = torch.zeros(1, dtype=torch.float32, device="cuda")
    ids = torch.full((B, K, s), -7, dtype=torch.int32, device="cuda")
    rc = mv.lib.medusa_heads_topk_noalloc(mv._ptr(h), mv._ptr(h), mv._ptr(h), B, K, d, V, s,
                                          mv.F32, None, mv._ptr(ids), None, None)
    assert rc == -8
    torch.cuda.synchronize()
    assert bool((ids == -7).all())
