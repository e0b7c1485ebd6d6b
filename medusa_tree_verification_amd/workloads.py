"""Seeded synthetic inputs for the Medusa verify step.

This module only *makes inputs*: random tensors, candidate trees and planted
verification logits.  It holds none of the verify step's arithmetic (no head
FFN, no top-s, no attention, no acceptance rule) and imports neither the HIP
library nor the CPU oracle, so both sides can consume the same bytes.

Workload shapes follow the method's description in "Medusa: Simple LLM
Inference Acceleration Framework with Multiple Decoding Heads" (paper
explainer page, sections on the head architecture, tree attention and
implementation notes): K heads on the last hidden state, top-s per head with
s = 3 recommended, a 4-deep tree with 63 candidates plus the root, and
Vicuna/Llama-7B-class sizes (d = 4096, V = 32000).

Random streams: every tensor is drawn from NumPy PCG64 seeded with
SeedSequence([1000*config_id + stream_id, chunk]) so that large tensors can be
generated in parallel chunks of CHUNK elements with a result that does not
depend on the thread count.  Stream ids:
 1 hidden, 2 W1, 3 W2, 4 q, 5 k_cache, 6 v_cache, 7 k_tree, 8 v_tree,
 9 prefix lengths, 10 verification logits (noise), 11 planting decisions,
 12 synthetic candidate-id table, 13 sampling uniforms, 14 LM head,
 15 tree-token embeddings h0, 16 final norm gain, and for the forward's
 block l: 200 + 8l + j with j = 0 gain, 1 Wq, 2 Wk, 3 Wv, 4 Wo, 5 k cache,
 6 v cache (l < 100).
bf16 tensors are drawn in fp32 and rounded to bf16 (round-to-nearest-even)
and are returned as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import itertools
import os
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk
# A re-drawn sequence row (hidden state) or re-planted logits row uses the
# stream's seed plus k * RESEED_STRIDE for its k-th re-draw (k >= 1).
RESEED_STRIDE = 100000

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    """One verify-step workload.  Sizes are per step on one GPU."""
    cid: int                 # seed namespace
    name: str
    dtype: str               # F32 or BF16 for every tensor of the step
    B: int                   # sequences in the batch
    K: int                   # Medusa heads (= maximum tree depth)
    d: int                   # hidden size
    V: int                   # vocabulary size
    s: int                   # candidates kept per head
    Hq: int                  # query heads
    Hkv: int                 # key/value heads (GQA when Hkv < Hq)
    dh: int                  # head dimension
    L_lo: int                # prefix length range [L_lo, L_hi] (uniform, inclusive)
    L_hi: int
    tree: str                # "full" or "pruned"
    T: int                   # tree nodes including the root
    rates: Tuple[Fraction, ...]  # per-depth acceptance-rate model (tree pruning + planting)
    mode: str                # "greedy" or "typical"
    temperature: float = 1.0
    eps: float = 0.09
    delta: float = 0.6

    @property
    def Lcap(self) -> int:
        return self.L_hi

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.dh))


def _fr(*xs: str) -> Tuple[Fraction, ...]:
    return tuple(Fraction(x) for x in xs)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload(1, "tiny_fp32", F32, B=1, K=3, d=256, V=1000, s=2, Hq=4, Hkv=4, dh=64,
                 L_lo=128, L_hi=128, tree="full", T=15, rates=_fr("0.6", "0.4", "0.3"),
                 mode="greedy"),
        Workload(2, "llama7b_b1", BF16, B=1, K=4, d=4096, V=32000, s=3, Hq=32, Hkv=32, dh=128,
                 L_lo=2048, L_hi=2048, tree="pruned", T=64,
                 rates=_fr("0.6", "0.4", "0.3", "0.2"), mode="greedy"),
        Workload(3, "ragged_b16_gqa_typical", BF16, B=16, K=4, d=4096, V=32000, s=3, Hq=32, Hkv=8,
                 dh=128, L_lo=512, L_hi=4096, tree="pruned", T=64,
                 rates=_fr("0.6", "0.4", "0.3", "0.2"), mode="typical", temperature=1.0),
        Workload(4, "long_ctx_32k", BF16, B=4, K=4, d=4096, V=32000, s=3, Hq=32, Hkv=8, dh=128,
                 L_lo=32768, L_hi=32768, tree="full", T=121,
                 rates=_fr("0.6", "0.4", "0.3", "0.2"), mode="greedy"),
        Workload(5, "large_vocab_typical", BF16, B=8, K=5, d=4096, V=128256, s=3, Hq=32, Hkv=8,
                 dh=128, L_lo=1024, L_hi=8192, tree="pruned", T=256,
                 rates=_fr("0.6", "0.4", "0.3", "0.2", "0.1"), mode="typical", temperature=0.7),
    ]
}

WORKLOAD_ORDER = ["tiny_fp32", "llama7b_b1", "ragged_b16_gqa_typical", "long_ctx_32k",
                  "large_vocab_typical"]


# --------------------------------------------------------------------------
# random tensors
# --------------------------------------------------------------------------
def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, chunk])))


def normal_tensor(seed: int, shape: Sequence[int], std: float, dtype: str) -> np.ndarray:
    """N(0, std^2) tensor, generated in seeded chunks; uint16 bits for bf16."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        a = _rng(seed, c).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        if dtype == BF16:
            b = a.view(np.uint32)
            b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
            b >>= np.uint32(16)
            out[lo:hi] = b
        else:
            out[lo:hi] = a

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(tuple(shape))


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float64 values (exact)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def encode(a: np.ndarray, dtype: str) -> np.ndarray:
    """float values -> stored tensor (fp32, or bf16 bits by nearest-even)."""
    a32 = np.asarray(a, dtype=np.float32)
    return f32_to_bf16_bits(a32) if dtype == BF16 else a32.copy()


# --------------------------------------------------------------------------
# candidate trees
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Tree:
    """A candidate tree in canonical order (depth, then rank tuple).

    paths[n] is node n's tuple of per-depth candidate ranks (empty for the
    root); parent[n] is the index of paths[n][:-1] (-1 for the root).
    """
    paths: List[Tuple[int, ...]]
    parent: np.ndarray  # int32 [T]

    @property
    def T(self) -> int:
        return len(self.paths)


def tree_from_paths(paths: Sequence[Tuple[int, ...]]) -> Tree:
    paths = sorted(set(tuple(p) for p in paths), key=lambda p: (len(p), p))
    if not paths or paths[0] != ():
        paths = [()] + [p for p in paths if p != ()]
    index = {p: i for i, p in enumerate(paths)}
    parent = np.full(len(paths), -1, dtype=np.int32)
    for i, p in enumerate(paths):
        if p:
            if p[:-1] not in index:
                raise ValueError(f"path {p} has no parent in the tree")
            parent[i] = index[p[:-1]]
    return Tree(list(paths), parent)


def full_product_tree(K: int, s: int) -> Tree:
    """Every rank tuple of length 0..K with entries < s (the uncut product)."""
    paths = [()]
    for depth in range(1, K + 1):
        paths += list(itertools.product(range(s), repeat=depth))
    return tree_from_paths(paths)


def pruned_tree(rates: Sequence[Fraction], s: int, T: int) -> Tree:
    """Cut the K-level product of top-s lists down to T nodes (root included).

    A head-j candidate of rank r is taken to be right with probability
    a_j (1 - a_j)^r (a geometric rank model built on the per-head rates); a
    node's score is the product along its path.  The root plus the T-1
    best-scoring nodes are kept, ties going to (shallower, lexicographically
    smaller rank tuple).  Scores fall strictly along every path and with
    rank, so the kept set is closed under taking parents and lower-ranked
    siblings.  Exact rational arithmetic keeps the cut free of rounding.
    """
    K = len(rates)
    scored = []
    for depth in range(1, K + 1):
        for tup in itertools.product(range(s), repeat=depth):
            sc = Fraction(1)
            for j, r in enumerate(tup):
                a = Fraction(rates[j])
                sc *= a * (1 - a) ** r
            scored.append((-sc, depth, tup))
    scored.sort()
    keep = [t for _, _, t in scored[: T - 1]]
    return tree_from_paths([()] + keep)


def random_tree(seed: int, T: int, K: int, s: int) -> Tree:
    """A random rank-closed tree with T nodes, depth <= K, <= s children each."""
    rng = _rng(seed)
    paths = [()]
    children: Dict[Tuple[int, ...], int] = {(): 0}
    while len(paths) < T:
        cands = [p for p in paths if len(p) < K and children[p] < s]
        if not cands:
            break
        p = cands[int(rng.integers(len(cands)))]
        c = p + (children[p],)
        children[p] += 1
        children[c] = 0
        paths.append(c)
    return tree_from_paths(paths)


def chain_tree(K: int) -> Tree:
    return tree_from_paths([tuple([0] * d) for d in range(K + 1)])


def workload_tree(wl: Workload) -> Tree:
    if wl.tree == "full":
        t = full_product_tree(wl.K, wl.s)
    else:
        t = pruned_tree(wl.rates, wl.s, wl.T)
    assert t.T == wl.T, (wl.name, t.T)
    return t


# --------------------------------------------------------------------------
# per-stage inputs
# --------------------------------------------------------------------------
def redrawn_row(seed: int, row: int, k: int, n: int, std: float, dtype: str) -> np.ndarray:
    """Row `row` of a tensor drawn from stream `seed`, re-drawn for the k-th
    time (k >= 1): N(0, std^2) from SeedSequence([seed + k*RESEED_STRIDE, row])."""
    a = _rng(seed + k * RESEED_STRIDE, row).standard_normal(n, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return encode(a, dtype)


def heads_inputs(wl: Workload, reseed: Optional[Dict[int, int]] = None) -> Dict[str, np.ndarray]:
    """hidden, W1, W2 of the workload.  reseed maps a sequence b to its
    re-draw count k: hidden[b] then comes from redrawn_row(stream 1, b, k)."""
    base = 1000 * wl.cid
    hidden = normal_tensor(base + 1, (wl.B, wl.d), 1.0, wl.dtype)
    for b, k in sorted((reseed or {}).items()):
        if k > 0:
            hidden[b] = redrawn_row(base + 1, b, k, wl.d, 1.0, wl.dtype)
    return {
        "hidden": hidden,
        "w1": normal_tensor(base + 2, (wl.K, wl.d, wl.d), 0.02, wl.dtype),
        "w2": normal_tensor(base + 3, (wl.K, wl.V, wl.d), 0.02, wl.dtype),
    }


def prefix_lengths(wl: Workload, seed_base: Optional[int] = None) -> np.ndarray:
    base = 1000 * wl.cid if seed_base is None else seed_base
    if wl.L_lo == wl.L_hi:
        return np.full(wl.B, wl.L_lo, dtype=np.int32)
    return _rng(base + 9).integers(wl.L_lo, wl.L_hi + 1, size=wl.B).astype(np.int32)


def attention_inputs(wl: Workload, T: Optional[int] = None) -> Dict[str, np.ndarray]:
    base = 1000 * wl.cid
    T = wl.T if T is None else T
    B, Hq, Hkv, dh, Lcap = wl.B, wl.Hq, wl.Hkv, wl.dh, wl.Lcap
    return {
        "q": normal_tensor(base + 4, (B, Hq, T, dh), 1.0, wl.dtype),
        "k_cache": normal_tensor(base + 5, (B, Hkv, Lcap, dh), 1.0, wl.dtype),
        "v_cache": normal_tensor(base + 6, (B, Hkv, Lcap, dh), 1.0, wl.dtype),
        "k_tree": normal_tensor(base + 7, (B, Hkv, T, dh), 1.0, wl.dtype),
        "v_tree": normal_tensor(base + 8, (B, Hkv, T, dh), 1.0, wl.dtype),
        "prefix_len": prefix_lengths(wl),
    }


def candidate_table(seed: int, B: int, K: int, s: int, V: int) -> np.ndarray:
    """Synthetic per-head candidate ids [B][K][s], distinct within (b, head)."""
    rng = _rng(seed)
    out = np.empty((B, K, s), dtype=np.int32)
    for b in range(B):
        for k in range(K):
            out[b, k] = rng.choice(V, size=s, replace=False)
    return out


def path_tokens(tree: Tree, table: np.ndarray) -> np.ndarray:
    """Token each node carries under the generator's own construction:
    node with rank tuple p holds table[b][len(p)-1][p[-1]]; the root gets -1."""
    B = table.shape[0]
    out = np.full((B, tree.T), -1, dtype=np.int32)
    for n, p in enumerate(tree.paths):
        if p:
            out[:, n] = table[:, len(p) - 1, p[-1]]
    return out


def _children(tree: Tree) -> Dict[int, List[int]]:
    kids: Dict[int, List[int]] = {}
    for n in range(1, tree.T):
        kids.setdefault(int(tree.parent[n]), []).append(n)
    return kids


def _plant_row(wl: Workload, tree: Tree, row: np.ndarray, n: int, ch: List[int],
               child_tok: List[int], rng: np.random.Generator) -> None:
    """Plant the children of internal node n into its fp32 noise row (in place)."""
    V = wl.V
    depth = len(tree.paths[n])
    a = float(wl.rates[min(depth, len(wl.rates) - 1)])
    ranks = [tree.paths[c][-1] for c in ch]
    if wl.mode == "greedy":
        probs = [a * (1 - a) ** r for r in ranks]
        u = rng.random()
        pick = -1
        acc = 0.0
        for i, p in enumerate(probs):
            acc += p
            if u < acc:
                pick = i
                break
        if pick >= 0:
            tok = child_tok[pick]
        else:
            tok = int(rng.integers(V))
            while tok in child_tok:
                tok = int(rng.integers(V))
        row[tok] = row.max() + rng.uniform(0.5, 1.5)
    else:
        peak = rng.uniform(11.0, 14.5)
        accept = [rng.random() < a * (1 - a) ** r for r in ranks]
        if accept and accept[0] and ranks[0] == 0:
            peak_tok = child_tok[0]
        else:
            peak_tok = int(rng.integers(V))
            while peak_tok in child_tok:
                peak_tok = int(rng.integers(V))
        row[peak_tok] = peak
        for i, t in enumerate(child_tok):
            if accept[i] and t != peak_tok:
                row[t] = peak - rng.uniform(0.3, 1.5)
        row *= np.float32(wl.temperature)


def replanted_row(wl: Workload, tree: Tree, tokens: np.ndarray, b: int, n: int, k: int,
                  seed_base: Optional[int] = None) -> np.ndarray:
    """Logits row (b, n) of an internal node n, re-planted for the k-th time
    (k >= 1): fresh noise and planting draws from streams 10 and 11 at
    seed + k*RESEED_STRIDE, row index b*T + n.  Returned in stored form."""
    base = 1000 * wl.cid if seed_base is None else seed_base
    T = tree.T
    ch = _children(tree)[n]
    idx = b * T + n
    row = _rng(base + 10 + k * RESEED_STRIDE, idx).standard_normal(wl.V, dtype=np.float32)
    _plant_row(wl, tree, row, n, ch, [int(tokens[b, c]) for c in ch],
               _rng(base + 11 + k * RESEED_STRIDE, idx))
    return encode(row, wl.dtype) if wl.dtype == BF16 else row


def verify_logits(wl: Workload, tree: Tree, tokens: np.ndarray,
                  seed_base: Optional[int] = None,
                  replant: Optional[Dict[Tuple[int, int], int]] = None) -> np.ndarray:
    """Verification logits [B][T][V] with candidates planted to be accepted at
    roughly the per-depth rates (a geometric model over sibling ranks).

    greedy: row noise N(0,1); one token per internal row is lifted to
      max(row) + U(0.5, 1.5): a child (chosen with prob a(1-a)^rank each) or
      otherwise a random non-child token.
    typical: tempered noise N(0,1) (stored as T*z); a peak token lifted to a
      height U(11, 14.5) in tempered units, which spreads the row entropy
      over roughly 0.4-5 nats at V = 32000..128256; children drawn as
      "accept" get a logit U(0.3, 1.5) below the peak (the rank-0 one may
      become the peak itself), the others keep their noise value.
    Leaf rows are plain noise.  replant maps (b, n) of an internal node to
    its re-plant count k: that row is then replanted_row(..., k).
    """
    base = 1000 * wl.cid if seed_base is None else seed_base
    B, T, V = wl.B, tree.T, wl.V
    noise = normal_tensor(base + 10, (B, T, V), 1.0, F32)
    rng = _rng(base + 11)
    kids = _children(tree)
    tau = float(wl.temperature)
    for b in range(B):
        for n, ch in kids.items():
            _plant_row(wl, tree, noise[b, n], n, ch, [int(tokens[b, c]) for c in ch], rng)
        if wl.mode == "typical":
            # leaf rows: same tempered scale as the internal ones
            for n in range(T):
                if n not in kids:
                    noise[b, n] *= np.float32(tau)
    out = encode(noise, wl.dtype) if wl.dtype == BF16 else noise
    for (b, n), k in sorted((replant or {}).items()):
        if k > 0:
            out[b, n] = replanted_row(wl, tree, tokens, b, n, k, base)
    return out


def forward_inputs(wl: Workload, N: int, T: Optional[int] = None,
                   seed_base: Optional[int] = None) -> Dict[str, object]:
    """Random-init weights and caches of N pre-norm attention blocks of the
    workload's shape plus its LM head, and embeddings h0 [B][T][d] of the
    tree tokens.  Projections ~ N(0, 1/fan_in), norm gains ~ N(1, 0.1^2),
    LM head ~ N(0, 0.02^2) (the heads' weight scale), h0 and the caches
    (keys taken as already rotated) ~ N(0, 1)."""
    if N > 100:
        raise ValueError("at most 100 blocks have their own seed streams")
    base = 1000 * wl.cid if seed_base is None else seed_base
    T = wl.T if T is None else T
    B, d, Hq, Hkv, dh, dt = wl.B, wl.d, wl.Hq, wl.Hkv, wl.dh, wl.dtype

    def gain(seed: int) -> np.ndarray:
        return encode(1.0 + normal_tensor(seed, (d,), 0.1, F32), dt)

    layers = []
    for l in range(N):
        sb = base + 200 + 8 * l
        layers.append({
            "g": gain(sb),
            "wq": normal_tensor(sb + 1, (Hq * dh, d), float(1 / np.sqrt(d)), dt),
            "wk": normal_tensor(sb + 2, (Hkv * dh, d), float(1 / np.sqrt(d)), dt),
            "wv": normal_tensor(sb + 3, (Hkv * dh, d), float(1 / np.sqrt(d)), dt),
            "wo": normal_tensor(sb + 4, (d, Hq * dh), float(1 / np.sqrt(Hq * dh)), dt),
        })
    return {
        "h0": normal_tensor(base + 15, (B, T, d), 1.0, dt),
        "layers": layers,
        "g_final": gain(base + 16),
        "w_lm": normal_tensor(base + 14, (wl.V, d), 0.02, dt),
        "k_caches": [normal_tensor(base + 205 + 8 * l, (B, Hkv, wl.Lcap, dh), 1.0, dt)
                     for l in range(N)],
        "v_caches": [normal_tensor(base + 206 + 8 * l, (B, Hkv, wl.Lcap, dh), 1.0, dt)
                     for l in range(N)],
        "prefix_len": prefix_lengths(wl, base),
    }
