"""GPU parity: medusa_sample_token (inversion sampling) against the oracle.

The kernel sums in fp32, so its distribution function is the oracle's
(fp64) one to within about 1e-6.  Random uniforms are re-drawn while they lie
within TOL of a boundary of the oracle's token interval, so that the drawn
token has one right answer and is compared exactly.  Uniforms placed on a
boundary on purpose (0 and the largest float below 1) are checked for a
token whose oracle interval holds u to within TOL."""
import numpy as np
import pytest
import torch

import oracle
from medusa_tree_verification_amd import workloads as W
from tests.util import Canaries, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _gpu(logits, rows, u, tau):
    from medusa_tree_verification_amd import binding as mv
    cz = Canaries()
    tok = cz.empty((len(u),), torch.int32)
    mv.medusa_sample_token(to_dev(logits), to_dev(np.asarray(rows, np.int32)),
                           to_dev(np.asarray(u, np.float32)), tau, token=tok)
    cz.check()
    return tok.cpu().numpy()


def _near(ref, u, b):
    return u[b] - ref["cdf_lo"][b] <= TOL or ref["cdf_hi"][b] - u[b] <= TOL


def _guard_u(logits, rows, u, tau, dtype, rng, fixed=()):
    """Re-draw the uniforms (other than the fixed ones) that lie within TOL of
    a boundary of the oracle's token interval."""
    u = np.asarray(u, np.float32).copy()
    for _ in range(64):
        ref = oracle.sample_token(logits, rows, u.astype(np.float64), tau, dtype, want_cdf=True)
        bad = [b for b in range(len(u)) if b not in fixed and ref["token"][b] >= 0
               and _near(ref, u.astype(np.float64), b)]
        if not bad:
            return u, ref
        for b in bad:
            u[b] = np.float32(rng.random())
    raise RuntimeError("uniforms not separated from the boundaries")


def _check(g, ref, u, fixed=()):
    u = np.asarray(u, np.float64)
    for b in range(len(u)):
        if ref["token"][b] < 0:
            assert g[b] == -1
            continue
        if b not in fixed:
            assert g[b] == ref["token"][b], (b, g[b], ref["token"][b], u[b])
            continue
        t = int(g[b])
        assert 0 <= t < ref["cdf"].shape[1], (b, t)
        lo_t = ref["cdf"][b, t - 1] if t > 0 else 0.0
        hi_t = ref["cdf"][b, t]
        assert lo_t <= u[b] + TOL and hi_t >= u[b] - TOL, (b, t, u[b], lo_t, hi_t)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 1000, 32000, 128256])
def test_sample_random(dtype, V):
    rng = np.random.default_rng(V + (dtype == "f32"))
    B, T = 24, 3
    x = (rng.standard_normal((B, T, V)) * 3).astype(np.float32)
    logits = W.encode(x.astype(np.float64), dtype)
    rows = rng.integers(0, T, B)
    u = rng.random(B).astype(np.float32)
    u[0], u[1] = 0.0, np.nextafter(np.float32(1), np.float32(0))
    rows[2], u[3] = T, 1.0                                 # invalid row / uniform -> -1
    for tau in (0.7, 1.0):
        ug, ref = _guard_u(logits, rows, u, tau, dtype, rng, fixed=(0, 1))
        _check(_gpu(logits, rows, ug, tau), ref, ug, fixed=(0, 1))


def test_sample_stratified_counts():
    """Identical rows and stratified uniforms: token counts within 2 of N p."""
    rng = np.random.default_rng(8)
    V, N, tau = 50, 4096, 0.8
    row = (rng.standard_normal(V) * 2).astype(np.float32)
    x = np.broadcast_to(row, (N, 1, V)).copy()
    u = ((np.arange(N) + 0.5) / N).astype(np.float32)
    g = _gpu(x, np.zeros(N, np.int32), u, tau)
    p = np.exp(row / tau - (row / tau).max())
    p /= p.sum()
    cnt = np.bincount(g, minlength=V)
    assert np.all(np.abs(cnt - N * p) <= 2.0), np.abs(cnt - N * p).max()


def test_sample_best_rows_of_a_workload():
    """Rows from tree_accept's best nodes on the large-vocabulary workload."""
    from medusa_tree_verification_amd import binding as mv
    wl = W.WORKLOADS["large_vocab_typical"]
    t = W.workload_tree(wl)
    ids = W.candidate_table(1000 * wl.cid + 12, wl.B, wl.K, wl.s, wl.V)
    logits = W.verify_logits(wl, t, W.path_tokens(t, ids))
    acc = mv.tree_accept(to_dev(logits), to_dev(ids), t.parent, mv.TYPICAL, wl.temperature)
    rows = acc["best_node"].cpu().numpy()
    rng = np.random.default_rng(2)
    u, ref = _guard_u(logits, rows, rng.random(wl.B), wl.temperature, wl.dtype, rng)
    g = _gpu(logits, rows, u, wl.temperature)
    _check(g, ref, u)
