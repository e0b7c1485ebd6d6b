"""CPU oracle of the Medusa verify step -- TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check and the bench's CPU-baseline leg may
import this package.  It wraps the plain fp64 C reference in
medusa_oracle.c (built with gcc, OpenMP over independent outputs) with NumPy
in/out.  Nothing here is shared with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "medusa_oracle.c")
_LIB = os.path.join(_HERE, "libmedusa_oracle.so")

DTYPE_CODE = {"f32": 0, "bf16": 1}
MODE_CODE = {"greedy": 0, "typical": 1, "typical_loglik": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library in place (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    """The oracle library; MEDUSA_ORACLE_LIB names another build of the same
    source (the sanitizer build of the CPU tests)."""
    global _lib
    if _lib is None:
        path = os.environ.get("MEDUSA_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        L.oracle_heads_topk.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P]
        L.oracle_tree.argtypes = [P, P, I, I, I, P, P, P]
        L.oracle_tree_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, P, I, P]
        L.oracle_tree_accept.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, D, D,
                                         P, P, P, P, P, P, P, P, P]
        L.oracle_num_threads.argtypes = []
        for f in ("oracle_heads_topk", "oracle_tree", "oracle_tree_attention",
                  "oracle_tree_accept", "oracle_num_threads"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: np.ndarray, dt) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dt)


def _stored(a: np.ndarray, dtype: str) -> np.ndarray:
    return _c(a, np.uint16 if dtype == "bf16" else np.float32)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def heads_topk(hidden, w1, w2, s: int, dtype: str) -> Dict[str, np.ndarray]:
    hidden, w1, w2 = (_stored(x, dtype) for x in (hidden, w1, w2))
    B, d = hidden.shape
    K, V = w2.shape[0], w2.shape[1]
    z = np.empty((B, K, d), np.float64)
    logits = np.empty((B, K, V), np.float64)
    ids = np.empty((B, K, s), np.int32)
    vals = np.empty((B, K, s), np.float64)
    rc = lib().oracle_heads_topk(_p(hidden), _p(w1), _p(w2), B, K, d, V, s, DTYPE_CODE[dtype],
                                 _p(z), _p(logits), _p(ids), _p(vals))
    _check(rc, "oracle_heads_topk")
    return {"z": z, "logits": logits, "topk_ids": ids, "topk_vals": vals}


def tree(parent, K: int, s: int, node_rank=None) -> Dict[str, np.ndarray]:
    parent = _c(parent, np.int32)
    T = parent.shape[0]
    nr = None if node_rank is None else _c(node_rank, np.int32)
    W = (T + 63) // 64
    depth = np.empty(T, np.int32)
    rank = np.empty(T, np.int32)
    mask = np.empty((T, W), np.uint64)
    rc = lib().oracle_tree(_p(parent), _p(nr), T, K, s, _p(depth), _p(rank), _p(mask))
    _check(rc, "oracle_tree")
    return {"depth": depth, "rank": rank, "mask": mask}


def tree_attention(q, k_cache, v_cache, prefix_len, k_tree, v_tree, parent, scale: float,
                   dtype: str, rows=None) -> np.ndarray:
    """Returns [B][Hq][T][dh] fp64, or [nrows][dh] when rows (n x 3) is given."""
    q, k_cache, v_cache, k_tree, v_tree = (_stored(x, dtype)
                                           for x in (q, k_cache, v_cache, k_tree, v_tree))
    prefix_len = _c(prefix_len, np.int32)
    parent = _c(parent, np.int32)
    B, Hq, T, dh = q.shape
    Hkv, Lcap = k_cache.shape[1], k_cache.shape[2]
    if rows is not None:
        rows = _c(rows, np.int32).reshape(-1, 3)
        out = np.empty((rows.shape[0], dh), np.float64)
        nrows = rows.shape[0]
    else:
        out = np.empty((B, Hq, T, dh), np.float64)
        nrows = 0
    rc = lib().oracle_tree_attention(_p(q), _p(k_cache), _p(v_cache), _p(prefix_len), _p(k_tree),
                                     _p(v_tree), _p(parent), B, Hq, Hkv, Lcap, dh, T, float(scale),
                                     DTYPE_CODE[dtype], _p(rows), nrows, _p(out))
    _check(rc, "oracle_tree_attention")
    return out


def tree_accept(logits, topk_ids, parent, dtype: str, mode: str, temperature: float = 1.0,
                eps: float = 0.09, delta: float = 0.6, node_rank=None) -> Dict[str, np.ndarray]:
    logits = _stored(logits, dtype)
    topk_ids = _c(topk_ids, np.int32)
    parent = _c(parent, np.int32)
    nr = None if node_rank is None else _c(node_rank, np.int32)
    B, T, V = logits.shape
    K, s = topk_ids.shape[1], topk_ids.shape[2]
    out = {
        "accept_len": np.empty(B, np.int32),
        "best_node": np.empty(B, np.int32),
        "accepted_tokens": np.empty((B, K), np.int32),
        "node_tokens": np.empty((B, T), np.int32),
        "next_token": np.empty(B, np.int32),
        "valid": np.empty((B, T), np.uint8),
        "ratio": np.empty((B, T), np.float64),
        "entropy": np.empty((B, T), np.float64),
        "score": np.empty((B, T), np.float64),
    }
    rc = lib().oracle_tree_accept(_p(logits), _p(topk_ids), _p(parent), _p(nr), B, T, V, K, s,
                                  DTYPE_CODE[dtype], MODE_CODE[mode], float(temperature),
                                  float(eps), float(delta), _p(out["accept_len"]),
                                  _p(out["best_node"]), _p(out["accepted_tokens"]),
                                  _p(out["node_tokens"]), _p(out["next_token"]), _p(out["valid"]),
                                  _p(out["ratio"]), _p(out["entropy"]), _p(out["score"]))
    _check(rc, "oracle_tree_accept")
    return out


def tree_commit_kv(k_cache, v_cache, prefix_len, k_tree, v_tree, best_node, parent
                   ) -> Dict[str, np.ndarray]:
    """Append each sequence's accepted path to its KV cache.

    After acceptance the sequence grows by the root token and the accepted
    candidates (page "Medusa：基于多Token预测的LLM推理加速", section 3.1, step 4
    of the decode loop: extend the sequence with the accepted tokens; the
    aiunderstanding page, section ディープダイブ: the longest matching prefix is
    kept).  Their keys and values were already computed by the tree pass, so
    the rows of the path root -> best_node[b] (depth order) are copied to cache
    positions L_b, L_b + 1, ... and the length advances by the path length.
    A sequence is left untouched (0 rows written) when L_b is outside
    [0, Lcap], best_node[b] is outside [0, T) or the path does not fit.
    Works on the stored element bits (any dtype): a pure copy.
    """
    k_cache, v_cache = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    L = _c(prefix_len, np.int32).copy()
    best_node = _c(best_node, np.int32)
    parent = _c(parent, np.int32)
    B, Hkv, Lcap, _ = k_cache.shape
    T = parent.shape[0]
    committed = np.zeros(B, np.int32)
    for b in range(B):
        best = int(best_node[b])
        if not (0 <= L[b] <= Lcap) or not (0 <= best < T):
            continue
        path = []
        a = best
        while a != -1:
            path.append(a)
            a = int(parent[a])
        path.reverse()                      # root first
        if L[b] + len(path) > Lcap:
            continue
        for j, node in enumerate(path):
            k_cache[b, :, L[b] + j, :] = k_tree[b, :, node, :]
            v_cache[b, :, L[b] + j, :] = v_tree[b, :, node, :]
        committed[b] = len(path)
        L[b] += len(path)
    return {"k_cache": k_cache, "v_cache": v_cache, "prefix_len": L, "committed": committed}


def sample_token(logits, rows, u, temperature: float, dtype: str,
                 want_cdf: bool = False) -> Dict[str, np.ndarray]:
    """The bonus token drawn from p = softmax(logits[b][rows[b]] / temperature)
    by inversion of its distribution function with the caller's uniform
    u[b] in [0, 1): the first token t whose cumulative probability
    P(<= t) exceeds u (page "Medusa：基于多Token预测的LLM推理加速", section 3.3:
    sampled verification draws from the tempered softmax).  fp64 throughout.
    Also returns, per sequence, P(< t) and P(<= t) of the drawn token; rows
    outside [0, T) or u outside [0, 1) give token -1.  With want_cdf, also
    the whole distribution function per sequence ([B][V], NaN rows where the
    token is -1)."""
    logits = _stored(logits, dtype)
    x = logits.astype(np.float32) if dtype == "f32" else \
        (logits.astype(np.uint32) << 16).view(np.float32)
    rows = _c(rows, np.int32)
    u = np.asarray(u, np.float64)
    B, T, V = x.shape
    tok = np.full(B, -1, np.int32)
    lo = np.zeros(B)
    hi = np.zeros(B)
    cdfs = np.full((B, V), np.nan) if want_cdf else None
    for b in range(B):
        r = int(rows[b])
        if not (0 <= r < T) or not (0.0 <= u[b] < 1.0):
            continue
        z = x[b, r].astype(np.float64) / temperature
        p = np.exp(z - z.max())
        cdf = np.cumsum(p) / p.sum()
        if want_cdf:
            cdfs[b] = cdf
        t = int(np.searchsorted(cdf, u[b], side="right"))   # first t with cdf[t] > u
        t = min(t, V - 1)
        tok[b] = t
        lo[b] = cdf[t - 1] if t > 0 else 0.0
        hi[b] = cdf[t]
    out = {"token": tok, "cdf_lo": lo, "cdf_hi": hi}
    if want_cdf:
        out["cdf"] = cdfs
    return out


def lm_head_argmax(hidden, w_lm, dtype: str) -> Dict[str, np.ndarray]:
    """Root token of the tree: the base model's own next token, the argmax
    of its LM head W_lm h on the last hidden state h (paper explainer page,
    section "Medusa Headのアーキテクチャ", its diagram: the original LM head
    gives x_{t+1}, Medusa head i gives x_{t+i+1}).  fp64 over the exactly
    decoded inputs; equal logits -> smaller id."""
    hidden = _stored(hidden, dtype)
    w_lm = _stored(w_lm, dtype)
    dec = (lambda a: a.astype(np.float64)) if dtype == "f32" else \
        (lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    logits = dec(hidden) @ dec(w_lm).T                      # [B][V]
    return {"logits": logits, "token": np.argmax(logits, axis=1).astype(np.int32)}


# ------------------------------------------------------------------
# Multi-layer synthetic verify forward (a second workload for the tree pass)
# ------------------------------------------------------------------
def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> the stored dtype and back: fp32 rounding, then (bf16) the
    upper 16 bits rounded to nearest-even."""
    f = np.asarray(x, np.float64).astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored bits (bf16) or fp32 values -> fp64."""
    a = _stored(a, dtype)
    if dtype == "f32":
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values already representable in dtype -> stored form."""
    f = np.asarray(x, np.float64).astype(np.float32)
    return f if dtype == "f32" else (f.view(np.uint32) >> 16).astype(np.uint16)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding on the last axis (dh), pairs (j, j + dh/2):
    angle pos * theta^(-2j/dh).  x: [..., n, dh] with pos broadcast to [..., n]."""
    dh = x.shape[-1]
    half = dh // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / dh)
    ang = np.asarray(pos, np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def verify_forward(h0, layers, g_final, w_lm, k_caches, v_caches, prefix_len, parent,
                   Hq: int, Hkv: int, dh: int, dtype: str, theta: float = 10000.0,
                   eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """N attention blocks over the tree tokens, then the LM head.

    The tree pass is one forward pass over all candidates with the tree mask
    (paper explainer page, tree-attention section); page
    "Medusa：基于多Token预测的LLM推理加速", section 5.3, runs the model once over
    the flattened tree and reads the logits of every position.  Each block:
    x = rmsnorm(h) g (rounded to dtype); q, k, v = x W^T (rounded after the
    rotary embedding of q and k at position L_b + depth(n)); o = tree
    attention over the block's cached prefix and the node's ancestors-or-self
    (rounded); h += o Wo^T (fp64 residual stream).  Finally
    logits = (rmsnorm(h) g_final, rounded) W_lm^T.  layers: a list of dicts
    with g, wq, wk, wv, wo in stored form; caches [B][Hkv][Lcap][dh] hold
    post-rotary keys.  Returns logits [B][T][V] and each block's tree k, v in
    stored form ([N][B][Hkv][T][dh])."""
    h = decode(h0, dtype)                         # [B][T][d]
    B, T, d = h.shape
    parent = _c(parent, np.int32)
    prefix_len = _c(prefix_len, np.int32)
    depth = tree(parent, T, max(T, 1))["depth"]
    Lcap = np.asarray(k_caches[0]).shape[2]
    pos = np.minimum(np.maximum(prefix_len, 0), Lcap)[:, None] + depth[None, :]   # [B][T]
    ks, vs = [], []
    for lw in layers:
        x = round_to(rmsnorm(h, decode(lw["g"], dtype), eps), dtype)
        q = (x @ decode(lw["wq"], dtype).T).reshape(B, T, Hq, dh).transpose(0, 2, 1, 3)
        k = (x @ decode(lw["wk"], dtype).T).reshape(B, T, Hkv, dh).transpose(0, 2, 1, 3)
        v = (x @ decode(lw["wv"], dtype).T).reshape(B, T, Hkv, dh).transpose(0, 2, 1, 3)
        q = round_to(rope(q, pos[:, None, :], theta), dtype)
        k = round_to(rope(k, pos[:, None, :], theta), dtype)
        v = round_to(v, dtype)
        kq, kk, kv = encode(q, dtype), encode(k, dtype), encode(v, dtype)
        ks.append(kk)
        vs.append(kv)
        o = tree_attention(kq, k_caches[len(ks) - 1], v_caches[len(vs) - 1], prefix_len, kk, kv,
                           parent, 1.0 / np.sqrt(dh), dtype)
        o = round_to(o, dtype).transpose(0, 2, 1, 3).reshape(B, T, Hq * dh)
        h = h + o @ decode(lw["wo"], dtype).T
    x = round_to(rmsnorm(h, decode(g_final, dtype), eps), dtype)
    logits = x @ decode(w_lm, dtype).T
    return {"logits": logits, "hidden": h, "k_tree": np.stack(ks) if ks else None,
            "v_tree": np.stack(vs) if vs else None}
