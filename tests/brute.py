"""Brute-force NumPy checks for the oracle (tiny inputs only).

These re-state what the verify step must produce in a different way from
the oracle: attention per candidate path as ordinary causal attention over
a flat sequence, tree relations from rank tuples instead of parent links,
and acceptance by enumerating every root-to-node path.
"""
from __future__ import annotations

import numpy as np
from scipy.special import softmax


def causal_attention_last(qs: np.ndarray, ks: np.ndarray, vs: np.ndarray, scale: float) -> np.ndarray:
    """Plain causal self-attention over a flat sequence (n x dh each); returns
    the output of the last position."""
    n = ks.shape[0]
    S = (qs @ ks.T) * scale
    causal = np.tril(np.ones((qs.shape[0], n), dtype=bool), k=n - qs.shape[0])
    S = np.where(causal, S, -np.inf)
    P = softmax(S, axis=-1)
    return (P @ vs)[-1]


def is_prefix(a, b) -> bool:
    return len(a) <= len(b) and tuple(b[: len(a)]) == tuple(a)


def path_nodes(paths, n):
    """Indices of the root..n path, found by matching rank-tuple prefixes."""
    target = paths[n]
    return sorted((m for m, p in enumerate(paths) if is_prefix(p, target)),
                  key=lambda m: len(paths[m]))


def accept_by_paths(paths, valid):
    """Deepest node whose whole root..node path is valid; lowest index wins."""
    best, best_d = 0, 0
    for n in range(1, len(paths)):
        if all(valid[m] for m in path_nodes(paths, n) if m != 0):
            if len(paths[n]) > best_d:
                best, best_d = n, len(paths[n])
    return best, best_d
