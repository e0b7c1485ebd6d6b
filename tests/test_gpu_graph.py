"""GPU: the verify step captured in a HIP graph replays like eager calls.

The library neither allocates, synchronizes nor clears memory with
hipMemsetAsync inside its calls, so a caller can capture a whole step
(heads, tree attention, acceptance, bonus-token draw; and the heads call
without a workspace) and replay it.  The graph is replayed several times,
with new inputs copied into its buffers, unrelated eager work and device
synchronizations between the replays, and every replay must equal bit for
bit the same calls run eagerly on the same inputs.  (The values themselves
are checked against the oracle by the other GPU tests.)"""
import numpy as np
import pytest

from medusa_tree_verification_amd import workloads as W
from tests.util import to_dev

pytestmark = pytest.mark.gpu


def _draw(seed, tree, B, K, d, V):
    return {"hidden": to_dev(W.normal_tensor(seed + 1, (B, d), 1.0, "bf16")),
            "logits": to_dev(W.normal_tensor(seed + 5, (B, tree.T, V), 2.0, "bf16")),
            "u": to_dev(np.random.default_rng(seed).random(B).astype(np.float32))}


def test_step_captured_in_a_graph_replays_like_eager():
    import torch
    from medusa_tree_verification_amd import binding as mv
    B, K, d, V, s = 8, 2, 1024, 20000, 4
    w1 = to_dev(W.normal_tensor(902, (K, d, d), 0.05, "bf16"))
    w2 = to_dev(W.normal_tensor(903, (K, V, d), 0.05, "bf16"))
    tree = W.random_tree(904, 21, K, s)
    wl = W.WORKLOADS["ragged_b16_gqa_typical"]   # pipelined attention plus the combine
    ax = {k: to_dev(v) for k, v in W.attention_inputs(wl).items()}
    at = W.workload_tree(wl)
    rows = torch.arange(B, dtype=torch.int32, device="cuda") % tree.T
    sets = [_draw(1100, tree, B, K, d, V), _draw(1200, tree, B, K, d, V)]

    # the buffers the graph reads (inputs) and writes (outputs), and the workspaces
    live = {k: v.clone() for k, v in sets[0].items()}
    i32 = dict(dtype=torch.int32, device="cuda")
    ws = {"heads": mv.workspace(mv.lib.medusa_heads_topk_workspace_bytes(B, K, d, V, s, mv.BF16),
                                "cuda"),
          "attn": mv.workspace(mv.lib.tree_attention_workspace_bytes(
              wl.B, wl.Hq, wl.Hkv, wl.Lcap, wl.dh, at.T, mv.BF16), "cuda"),
          "accept": mv.workspace(mv.lib.tree_accept_workspace_bytes(B, tree.T, V, K, s), "cuda")}

    def new_out():
        return {"ids": torch.empty((B, K, s), **i32),
                "vals": torch.empty((B, K, s), dtype=torch.float32, device="cuda"),
                "ids_na": torch.empty((B, K, s), **i32),
                "attn": torch.empty_like(ax["q"]),
                "acc": {k: torch.empty(sh, **i32) for k, sh in (
                    ("accept_len", (B,)), ("best_node", (B,)), ("accepted_tokens", (B, K)),
                    ("node_tokens", (B, tree.T)), ("next_token", (B,)))},
                "tok": torch.empty((B,), **i32)}

    def step(inp, o):
        mv.medusa_heads_topk(inp["hidden"], w1, w2, s, ws=ws["heads"],
                             out={"topk_ids": o["ids"], "topk_vals": o["vals"]})
        mv.medusa_heads_topk_noalloc(inp["hidden"], w1, w2, s, out={"topk_ids": o["ids_na"]})
        mv.tree_attention(ax["q"], ax["k_cache"], ax["v_cache"], ax["prefix_len"], ax["k_tree"],
                          ax["v_tree"], at.parent, wl.scale, ws=ws["attn"], out=o["attn"])
        mv.tree_accept(inp["logits"], o["ids"], tree.parent, mv.TYPICAL, 0.7, ws=ws["accept"],
                       out=o["acc"])
        mv.medusa_sample_token(inp["logits"], rows, inp["u"], 0.7, token=o["tok"])

    def flat(o):
        res = []
        for k in sorted(o):
            v = o[k]
            for t in ([v[j] for j in sorted(v)] if isinstance(v, dict) else [v]):
                res.append(t.contiguous().view(torch.uint8).cpu().numpy())
        return res

    # eager results for both input sets
    refs = []
    for inp in sets:
        o = new_out()
        step(inp, o)
        torch.cuda.synchronize()
        refs.append(flat(o))
    assert any(not np.array_equal(a, b) for a, b in zip(refs[0], refs[1]))

    # capture (after a warm-up on the capture stream, as torch asks)
    g_out = new_out()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(live, g_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(live, g_out)
    torch.cuda.synchronize()

    a = torch.randn(2048, 2048, device="cuda")
    for r, which in enumerate([0, 1, 1, 0, 1]):
        for k in live:
            live[k].copy_(sets[which][k])
        for v in (g_out["ids"], g_out["ids_na"], g_out["tok"]):
            v.fill_(-7)
        a = torch.mm(a, a) * 1e-3          # the program's own eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = flat(g_out)
        for i, (x, y) in enumerate(zip(got, refs[which])):
            assert np.array_equal(x, y), f"replay {r} (inputs {which}): output {i} differs"
        print(f"replay {r} (inputs {which}): identical to the eager calls", flush=True)
