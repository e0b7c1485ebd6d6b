"""CPU: the input guards (tests/guards.py) and the generator's re-draw paths."""
import dataclasses

import numpy as np

from medusa_tree_verification_amd import workloads as W
from tests import guards


def test_topk_margin_definition():
    row = np.array([0.0, 3.0, 1.0, 3.0 + 1e-9, -2.0])
    rms = np.sqrt(np.mean(row ** 2))
    assert abs(guards.topk_margin(row, 2) - 1e-9 / rms) < 1e-15
    assert abs(guards.topk_margin(row, 3) - 1e-9 / rms) < 1e-15
    assert guards.topk_margin(np.array([5.0]), 3) == np.inf


def test_g1_redraws_a_tied_sequence_and_the_generator_reproduces_it():
    """Two head rows that read single coordinates of z = h (W1 = 0): planting
    h0 == h1 ties them, so G1 must re-draw exactly that sequence, with the
    generator's k-th re-draw."""
    B, K, d, V, s = 3, 1, 128, 4, 1
    seed = 777
    hx = {"hidden": W.normal_tensor(seed, (B, d), 1.0, "f32"),
          "w1": np.zeros((K, d, d), np.float32),
          "w2": np.zeros((K, V, d), np.float32)}
    for v in range(V):
        hx["w2"][0, v, v] = 1.0
    hx["hidden"][1, :V] = 5.0          # rows 0..3 of sequence 1 all tie at the top
    ref, _, bumps = guards.guard_heads(hx, s, "f32",
                                       lambda b, k: W.redrawn_row(seed, b, k, d, 1.0, "f32"),
                                       "tie test")
    assert set(bumps) == {1}
    np.testing.assert_array_equal(hx["hidden"][1], W.redrawn_row(seed, 1, bumps[1], d, 1.0, "f32"))
    for b in range(B):
        assert guards.topk_margin(ref["logits"][b, 0], s + 1) >= guards.G_REL


def test_heads_inputs_reseed_replaces_only_that_row():
    wl = W.WORKLOADS["tiny_fp32"]
    a = W.heads_inputs(wl)
    b = W.heads_inputs(wl, reseed={0: 2})
    np.testing.assert_array_equal(b["hidden"][0], W.redrawn_row(1000 * wl.cid + 1, 0, 2, wl.d,
                                                                1.0, wl.dtype))
    assert not np.array_equal(a["hidden"][0], b["hidden"][0])
    np.testing.assert_array_equal(a["w2"], b["w2"])


def _small_typical():
    base = W.WORKLOADS["ragged_b16_gqa_typical"]
    return dataclasses.replace(base, cid=91, name="small_typical", B=3, V=300, T=15, K=3, s=2,
                               tree="full", rates=W._fr("0.6", "0.4", "0.3"))


def test_g2_guard_leaves_no_knife_edge_and_replant_reproduces():
    wl = _small_typical()
    t = W.full_product_tree(wl.K, wl.s)
    ids = W.candidate_table(5, wl.B, wl.K, wl.s, wl.V)
    logits, ref, replant = guards.guard_typical(wl, t, ids, "small typical")
    assert not guards.g2_bad(ref, t.parent)
    again = W.verify_logits(wl, t, W.path_tokens(t, ids), replant=replant)
    np.testing.assert_array_equal(again, logits)


def test_g2_detects_a_knife_edge():
    ref = {"ratio": np.array([[0.0, 1.0004, 0.5, 2.0], [0.0, 0.9, 1.1, 0.9995]])}
    parent = np.array([-1, 0, 0, 1])
    bad = guards.g2_bad(ref, parent)
    assert set(bad) == {(0, 0), (1, 1)}


def test_replanted_row_is_a_fresh_planting():
    wl = _small_typical()
    t = W.full_product_tree(wl.K, wl.s)
    ids = W.candidate_table(6, wl.B, wl.K, wl.s, wl.V)
    tok = W.path_tokens(t, ids)
    base = W.verify_logits(wl, t, tok)
    r1 = W.replanted_row(wl, t, tok, 1, 0, 1)
    r2 = W.replanted_row(wl, t, tok, 1, 0, 2)
    assert r1.shape == (wl.V,) and not np.array_equal(r1, r2)
    rp = W.verify_logits(wl, t, tok, replant={(1, 0): 1})
    np.testing.assert_array_equal(rp[1, 0], r1)
    rp[1, 0] = base[1, 0]
    np.testing.assert_array_equal(rp, base)
