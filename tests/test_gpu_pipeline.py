"""GPU: the three calls chained as one verify step (heads -> acceptance),
against the oracle fed the same inputs."""
import numpy as np
import pytest

import oracle
from medusa_tree_verification_amd import workloads as W
from tests.util import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_fp32", "llama7b_b1"])
def test_step_heads_feed_acceptance(name):
    from medusa_tree_verification_amd import binding as mv
    wl = W.WORKLOADS[name]
    t = W.workload_tree(wl)
    hx = W.heads_inputs(wl)
    ref_h = oracle.heads_topk(hx["hidden"], hx["w1"], hx["w2"], wl.s, wl.dtype)
    ids_ref = ref_h["topk_ids"]
    logits = W.verify_logits(wl, t, W.path_tokens(t, ids_ref))
    h = mv.medusa_heads_topk(to_dev(hx["hidden"]), to_dev(hx["w1"]), to_dev(hx["w2"]), wl.s)
    np.testing.assert_array_equal(h["topk_ids"].cpu().numpy(), ids_ref)
    acc = mv.tree_accept(to_dev(logits), h["topk_ids"], t.parent,
                         mv.GREEDY if wl.mode == "greedy" else mv.TYPICAL, wl.temperature)
    ref = oracle.tree_accept(logits, ids_ref, t.parent, wl.dtype, wl.mode, wl.temperature)
    for k in ("accept_len", "best_node", "accepted_tokens", "node_tokens", "next_token"):
        np.testing.assert_array_equal(acc[k].cpu().numpy(), ref[k])
    assert ref["accept_len"].max() > 0


def test_smoke_entry():
    import __graft_entry__
    __graft_entry__.smoke()
