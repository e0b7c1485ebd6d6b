"""Thin ctypes binding of libmedusa_verify.so (argument marshalling only).

Every step of the verify path runs in the HIP kernels behind the C ABI in
include/medusa_verify.h; these wrappers only turn torch tensors (device
memory) into pointers, allocate outputs/workspace with torch and pass the
current stream.  There is no other implementation: if the library is
missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmedusa_verify.so")

F32, BF16 = 0, 1
GREEDY, TYPICAL, TYPICAL_LOGLIK = 0, 1, 2

STATUS = {0: "MEDUSA_OK", -1: "MEDUSA_ERR_NULL", -2: "MEDUSA_ERR_SHAPE", -3: "MEDUSA_ERR_DTYPE",
          -4: "MEDUSA_ERR_TREE", -5: "MEDUSA_ERR_WORKSPACE", -6: "MEDUSA_ERR_PARAM",
          -7: "MEDUSA_ERR_LAUNCH", -8: "MEDUSA_ERR_SCRATCH"}

EXPORTS = ["medusa_heads_topk", "medusa_heads_topk_root", "medusa_heads_stage1",
           "medusa_heads_stage2", "medusa_heads_stage2_stream", "medusa_heads_stage2_merge",
           "medusa_heads_topk_workspace_bytes", "medusa_heads_topk_noalloc",
           "medusa_heads_topk_noalloc_max_scratch", "tree_attention", "tree_attention_workspace_bytes",
           "tree_accept", "tree_accept_workspace_bytes", "tree_commit_kv", "medusa_sample_token",
           "medusa_verify_forward", "medusa_verify_forward_workspace_bytes", "medusa_status_str",
           "medusa_abi_version"]
PROBE_EXPORTS = ["medusa_probe_sink_bytes", "medusa_probe_read", "medusa_probe_mfma",
                 "medusa_probe_mfma_flops", "medusa_probe_read_timed",
                 "medusa_probe_read_workgroups", "medusa_probe_clock_mhz"]


class MedusaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}: {status_str(code)}")
        self.code = code


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run medusa_tree_verification_amd/build.py "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.medusa_heads_topk.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P, Z, P]
    L.medusa_heads_topk_root.argtypes = [P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P, Z, P]
    L.medusa_heads_stage1.argtypes = [P, P, I, I, I, I, I, I, P, Z, P]
    L.medusa_heads_stage2.argtypes = [P, I, I, I, I, I, I, P, P, P, P, Z, P]
    L.medusa_heads_stage2_stream.argtypes = [P, I, I, I, I, I, I, P, P, Z, P]
    L.medusa_heads_stage2_merge.argtypes = [I, I, I, I, I, I, P, P, P, Z, P]
    L.medusa_heads_topk_workspace_bytes.argtypes = [I, I, I, I, I, I]
    L.medusa_heads_topk_workspace_bytes.restype = Z
    L.medusa_heads_topk_noalloc.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P]
    L.medusa_heads_topk_noalloc_max_scratch.argtypes = []
    L.medusa_heads_topk_noalloc_max_scratch.restype = Z
    L.tree_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, Z, P]
    L.tree_attention_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    L.tree_attention_workspace_bytes.restype = Z
    L.tree_accept.argtypes = [P, P, P, P, I, I, I, I, I, I, I, F, F, F, P, P, P, P, P, P, Z, P]
    L.tree_accept_workspace_bytes.argtypes = [I, I, I, I, I]
    L.tree_accept_workspace_bytes.restype = Z
    L.tree_commit_kv.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P]
    L.medusa_sample_token.argtypes = [P, P, P, I, I, I, I, F, P, P]
    D = ctypes.c_double
    L.medusa_verify_forward.argtypes = [P, I, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                        I, I, D, F, P, P, P, P, P, Z, P]
    L.medusa_verify_forward_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I]
    L.medusa_verify_forward_workspace_bytes.restype = Z
    L.medusa_status_str.argtypes = [I]
    L.medusa_status_str.restype = ctypes.c_char_p
    L.medusa_abi_version.restype = I
    L.medusa_probe_sink_bytes.argtypes = []
    L.medusa_probe_sink_bytes.restype = Z
    L.medusa_probe_read.argtypes = [P, Z, P, P]
    L.medusa_probe_read.restype = I
    L.medusa_probe_read_timed.argtypes = [P, Z, P, P, I, P]
    L.medusa_probe_read_timed.restype = I
    L.medusa_probe_read_workgroups.argtypes = []
    L.medusa_probe_read_workgroups.restype = I
    L.medusa_probe_clock_mhz.argtypes = []
    L.medusa_probe_clock_mhz.restype = ctypes.c_double
    L.medusa_probe_mfma.argtypes = [I, P, P]
    L.medusa_probe_mfma.restype = I
    L.medusa_probe_mfma_flops.argtypes = [I]
    L.medusa_probe_mfma_flops.restype = ctypes.c_double
    for f in ("medusa_heads_topk", "medusa_heads_topk_noalloc", "medusa_heads_topk_root",
              "medusa_heads_stage1",
              "medusa_heads_stage2", "medusa_heads_stage2_stream", "medusa_heads_stage2_merge",
              "tree_attention",
              "tree_accept", "tree_commit_kv", "medusa_sample_token", "medusa_verify_forward"):
        getattr(L, f).restype = I
    return L


lib = _load()


def status_str(code: int) -> str:
    return lib.medusa_status_str(int(code)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MedusaError(fn, rc)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def _host_i32(a: Optional[Sequence[int]]):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def workspace(nbytes: int, device) -> torch.Tensor:
    """A device byte buffer (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
def medusa_heads_topk(hidden: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, s: int, *,
                      want_logits: bool = False, ws: Optional[torch.Tensor] = None,
                      out: Optional[Dict[str, torch.Tensor]] = None,
                      stream=None) -> Dict[str, torch.Tensor]:
    for t, n in ((hidden, "hidden"), (w1, "w1"), (w2, "w2")):
        _need(t, n)
    B, d = hidden.shape
    K, V = w2.shape[0], w2.shape[1]
    dt = _dtype_code(hidden)
    dev = hidden.device
    if out is None:
        out = {"topk_ids": torch.empty((B, K, s), dtype=torch.int32, device=dev),
               "topk_vals": torch.empty((B, K, s), dtype=torch.float32, device=dev)}
        if want_logits:
            out["logits"] = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(lib.medusa_heads_topk_workspace_bytes(B, K, d, V, s, dt), dev)
    rc = lib.medusa_heads_topk(_ptr(hidden), _ptr(w1), _ptr(w2), B, K, d, V, s, dt,
                               _ptr(out.get("logits")), _ptr(out["topk_ids"]),
                               _ptr(out.get("topk_vals")), _ptr(ws), ws.numel(), _stream(stream))
    _check("medusa_heads_topk", rc)
    return out


def medusa_heads_topk_noalloc(hidden: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, s: int,
                              *, out: Dict[str, torch.Tensor],
                              stream=None) -> Dict[str, torch.Tensor]:
    """medusa_heads_topk with the library's static scratch instead of a
    workspace; the caller passes every output (out: topk_ids, and optionally
    topk_vals and logits), so this wrapper allocates nothing either."""
    for t, n in ((hidden, "hidden"), (w1, "w1"), (w2, "w2")):
        _need(t, n)
    B, d = hidden.shape
    K, V = w2.shape[0], w2.shape[1]
    rc = lib.medusa_heads_topk_noalloc(_ptr(hidden), _ptr(w1), _ptr(w2), B, K, d, V, s,
                                       _dtype_code(hidden), _ptr(out.get("logits")),
                                       _ptr(out["topk_ids"]), _ptr(out.get("topk_vals")),
                                       _stream(stream))
    _check("medusa_heads_topk_noalloc", rc)
    return out


def medusa_heads_stage1(hidden, w1, B, K, d, V, s, ws, stream=None) -> None:
    rc = lib.medusa_heads_stage1(_ptr(hidden), _ptr(w1), B, K, d, V, s, _dtype_code(hidden),
                                 _ptr(ws), ws.numel(), _stream(stream))
    _check("medusa_heads_stage1", rc)


def medusa_heads_stage2(w2, B, K, d, V, s, topk_ids, ws, topk_vals=None, logits=None,
                        stream=None) -> None:
    rc = lib.medusa_heads_stage2(_ptr(w2), B, K, d, V, s, _dtype_code(w2), _ptr(logits),
                                 _ptr(topk_ids), _ptr(topk_vals), _ptr(ws), ws.numel(),
                                 _stream(stream))
    _check("medusa_heads_stage2", rc)


def medusa_heads_stage2_stream(w2, B, K, d, V, s, ws, logits=None, stream=None) -> None:
    rc = lib.medusa_heads_stage2_stream(_ptr(w2), B, K, d, V, s, _dtype_code(w2), _ptr(logits),
                                        _ptr(ws), ws.numel(), _stream(stream))
    _check("medusa_heads_stage2_stream", rc)


def medusa_heads_stage2_merge(B, K, d, V, s, dtype_code, topk_ids, ws, topk_vals=None,
                              stream=None) -> None:
    rc = lib.medusa_heads_stage2_merge(B, K, d, V, s, int(dtype_code), _ptr(topk_ids),
                                       _ptr(topk_vals), _ptr(ws), ws.numel(), _stream(stream))
    _check("medusa_heads_stage2_merge", rc)


def tree_attention(q, k_cache, v_cache, prefix_len, k_tree, v_tree, parent, scale: float, *,
                   want_mask: bool = False, ws: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None, mask_out: Optional[torch.Tensor] = None,
                   stream=None):
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (prefix_len, "prefix_len"),
                 (k_tree, "k_tree"), (v_tree, "v_tree")):
        _need(t, n)
    B, Hq, T, dh = q.shape
    Hkv, Lcap = k_cache.shape[1], k_cache.shape[2]
    dt = _dtype_code(q)
    dev = q.device
    par, par_p = _host_i32(parent)
    if out is None:
        out = torch.empty_like(q)
    if want_mask and mask_out is None:
        mask_out = torch.empty((T, (T + 63) // 64), dtype=torch.int64, device=dev)
    if ws is None:
        ws = workspace(lib.tree_attention_workspace_bytes(B, Hq, Hkv, Lcap, dh, T, dt), dev)
    rc = lib.tree_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len), _ptr(k_tree),
                            _ptr(v_tree), par_p, B, Hq, Hkv, Lcap, dh, T, float(scale), dt,
                            _ptr(out), _ptr(mask_out), _ptr(ws), ws.numel(), _stream(stream))
    _check("tree_attention", rc)
    return (out, mask_out) if want_mask else out


def tree_accept(logits, topk_ids, parent, mode: int, temperature: float = 1.0, eps: float = 0.09,
                delta: float = 0.6, node_rank=None, *, ws: Optional[torch.Tensor] = None,
                out: Optional[Dict[str, torch.Tensor]] = None,
                stream=None) -> Dict[str, torch.Tensor]:
    _need(logits, "logits")
    _need(topk_ids, "topk_ids")
    B, T, V = logits.shape
    K, s = topk_ids.shape[1], topk_ids.shape[2]
    dt = _dtype_code(logits)
    dev = logits.device
    par, par_p = _host_i32(parent)
    nr, nr_p = _host_i32(node_rank)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {"accept_len": torch.empty(B, **i32), "best_node": torch.empty(B, **i32),
               "accepted_tokens": torch.empty((B, K), **i32),
               "node_tokens": torch.empty((B, T), **i32), "next_token": torch.empty(B, **i32)}
    if ws is None:
        ws = workspace(lib.tree_accept_workspace_bytes(B, T, V, K, s), dev)
    rc = lib.tree_accept(_ptr(logits), _ptr(topk_ids), par_p, nr_p, B, T, V, K, s, dt, int(mode),
                         float(temperature), float(eps), float(delta), _ptr(out["accept_len"]),
                         _ptr(out["best_node"]), _ptr(out["accepted_tokens"]),
                         _ptr(out.get("node_tokens")), _ptr(out.get("next_token")), _ptr(ws),
                         ws.numel(), _stream(stream))
    _check("tree_accept", rc)
    return out


def tree_commit_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, prefix_len: torch.Tensor,
                   k_tree: torch.Tensor, v_tree: torch.Tensor, best_node: torch.Tensor, parent,
                   committed: Optional[torch.Tensor] = None, stream=None) -> Optional[torch.Tensor]:
    """Append the accepted path's K/V rows to the caches (in place) and
    advance prefix_len (in place); returns `committed` if given."""
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (prefix_len, "prefix_len"),
                 (k_tree, "k_tree"), (v_tree, "v_tree"), (best_node, "best_node")):
        _need(t, n)
    B, Hkv, Lcap, dh = k_cache.shape
    T = k_tree.shape[2]
    par, par_p = _host_i32(parent)
    rc = lib.tree_commit_kv(_ptr(k_cache), _ptr(v_cache), _ptr(prefix_len), _ptr(k_tree),
                            _ptr(v_tree), _ptr(best_node), par_p, B, Hkv, Lcap, dh, T,
                            _dtype_code(k_cache), _ptr(committed), _stream(stream))
    _check("tree_commit_kv", rc)
    return committed


def medusa_sample_token(logits: torch.Tensor, rows: torch.Tensor, u: torch.Tensor,
                        temperature: float, token: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Bonus token per sequence drawn from softmax(logits[b][rows[b]] / temperature)
    by inversion with the uniforms u (device float32 [B])."""
    for t, n in ((logits, "logits"), (rows, "rows"), (u, "u")):
        _need(t, n)
    B, T, V = logits.shape
    if token is None:
        token = torch.empty(B, dtype=torch.int32, device=logits.device)
    rc = lib.medusa_sample_token(_ptr(logits), _ptr(rows), _ptr(u), B, T, V, _dtype_code(logits),
                                 float(temperature), _ptr(token), _stream(stream))
    _check("medusa_sample_token", rc)
    return token


def medusa_heads_topk_root(hidden: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor,
                           w_lm: torch.Tensor, s: int, *, ws: Optional[torch.Tensor] = None,
                           stream=None) -> Dict[str, torch.Tensor]:
    """The K heads' top-s plus the root token (argmax of the LM head w_lm on
    the hidden state), in one weight stream."""
    for t, n in ((hidden, "hidden"), (w1, "w1"), (w2, "w2"), (w_lm, "w_lm")):
        _need(t, n)
    B, d = hidden.shape
    K, V = w2.shape[0], w2.shape[1]
    dt = _dtype_code(hidden)
    dev = hidden.device
    out = {"topk_ids": torch.empty((B, K, s), dtype=torch.int32, device=dev),
           "topk_vals": torch.empty((B, K, s), dtype=torch.float32, device=dev),
           "root_token": torch.empty(B, dtype=torch.int32, device=dev),
           "root_val": torch.empty(B, dtype=torch.float32, device=dev)}
    if ws is None:
        ws = workspace(lib.medusa_heads_topk_workspace_bytes(B, K, d, V, s, dt), dev)
    rc = lib.medusa_heads_topk_root(_ptr(hidden), _ptr(w1), _ptr(w2), _ptr(w_lm), B, K, d, V, s,
                                    dt, None, _ptr(out["topk_ids"]), _ptr(out["topk_vals"]),
                                    _ptr(out["root_token"]), _ptr(out["root_val"]), _ptr(ws),
                                    ws.numel(), _stream(stream))
    _check("medusa_heads_topk_root", rc)
    return out


def _ptr_array(ts: Sequence[torch.Tensor], name: str):
    for i, t in enumerate(ts):
        _need(t, f"{name}[{i}]")
    arr = (ctypes.c_void_p * max(len(ts), 1))(*[t.data_ptr() for t in ts])
    return arr


def medusa_verify_forward(h0: torch.Tensor, layers: Sequence[Dict[str, torch.Tensor]],
                          g_final: torch.Tensor, w_lm: torch.Tensor,
                          k_caches: Sequence[torch.Tensor], v_caches: Sequence[torch.Tensor],
                          prefix_len: torch.Tensor, parent, Hq: int, Hkv: int, dh: int, *,
                          theta: float = 10000.0, eps: float = 1e-6, want_hidden: bool = False,
                          want_kv: bool = False, ws: Optional[torch.Tensor] = None,
                          out: Optional[Dict[str, torch.Tensor]] = None,
                          stream=None) -> Dict[str, torch.Tensor]:
    """Logits [B][T][V] (float32) of the tree tokens from N attention blocks
    (layers: dicts with g, wq, wk, wv, wo) and the LM head; optionally the
    final residual stream (hidden) and every block's tree k/v."""
    for t, n in ((h0, "h0"), (g_final, "g_final"), (w_lm, "w_lm"), (prefix_len, "prefix_len")):
        _need(t, n)
    B, T, d = h0.shape
    V = w_lm.shape[0]
    N = len(layers)
    Lcap = k_caches[0].shape[2] if N else 0
    dt = _dtype_code(h0)
    dev = h0.device
    par, par_p = _host_i32(parent)
    arrs = {k: _ptr_array([lw[k] for lw in layers], k) for k in ("g", "wq", "wk", "wv", "wo")}
    kc = _ptr_array(list(k_caches), "k_caches")
    vc = _ptr_array(list(v_caches), "v_caches")
    if out is None:
        out = {"logits": torch.empty((B, T, V), dtype=torch.float32, device=dev)}
        if want_hidden:
            out["hidden"] = torch.empty((B, T, d), dtype=torch.float32, device=dev)
        if want_kv and N:
            out["k_tree"] = torch.empty((N, B, Hkv, T, dh), dtype=h0.dtype, device=dev)
            out["v_tree"] = torch.empty((N, B, Hkv, T, dh), dtype=h0.dtype, device=dev)
    if ws is None:
        ws = workspace(lib.medusa_verify_forward_workspace_bytes(B, T, d, Hq, Hkv, dh, Lcap, V, dt),
                       dev)
    rc = lib.medusa_verify_forward(
        _ptr(h0), N, arrs["g"], arrs["wq"], arrs["wk"], arrs["wv"], arrs["wo"], _ptr(g_final),
        _ptr(w_lm), kc, vc, _ptr(prefix_len), par_p, B, T, d, Hq, Hkv, dh, Lcap, V, dt,
        float(theta), float(eps), _ptr(out["logits"]), _ptr(out.get("hidden")),
        _ptr(out.get("k_tree")), _ptr(out.get("v_tree")), _ptr(ws), ws.numel(), _stream(stream))
    _check("medusa_verify_forward", rc)
    return out


# ---------------------------------------------------------------------------
# peak probes (include/medusa_probes.h)
def probe_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """One linear 16-byte-load pass over buf (device)."""
    _need(buf, "buf")
    rc = lib.medusa_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                               _stream(stream))
    _check("medusa_probe_read", rc)


def probe_read_timed(buf: torch.Tensor, sink: torch.Tensor, stamps: torch.Tensor,
                     pattern: int = 0, stream=None) -> None:
    """A read pass (pattern 0: linear; 1: 8-row tiles of 8 KiB rows) that
    records every workgroup's start and end clock in stamps (device int32, 2
    per workgroup)."""
    _need(buf, "buf")
    _need(stamps, "stamps")
    if stamps.numel() * stamps.element_size() < 8 * lib.medusa_probe_read_workgroups():
        raise ValueError("stamps: 2 int32 per workgroup needed")
    rc = lib.medusa_probe_read_timed(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                     _ptr(stamps), int(pattern), _stream(stream))
    _check("medusa_probe_read_timed", rc)


def probe_mfma(iters: int, sink: torch.Tensor, stream=None) -> float:
    """Independent bf16 32x32x16 MFMA chains; returns the FLOPs of the call."""
    rc = lib.medusa_probe_mfma(int(iters), _ptr(sink), _stream(stream))
    _check("medusa_probe_mfma", rc)
    return float(lib.medusa_probe_mfma_flops(int(iters)))
