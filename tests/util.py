"""Shared helpers for the parity tests (no verify-step arithmetic here)."""
from __future__ import annotations

import numpy as np

from medusa_tree_verification_amd import workloads as W

CANARY_BYTE = 0xA5          # fill of the guard bands around GPU outputs
CANARY_BYTES = 4096         # guard band before and after each output


def to_dev(a: np.ndarray, dtype: str = None):
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy()


def normwise(gpu: np.ndarray, ref: np.ndarray, axes) -> np.ndarray:
    """max|gpu - ref| / max|ref| over the given axes."""
    num = np.abs(gpu.astype(np.float64) - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    return num / np.maximum(den, 1e-300)


class Canaries:
    """Device output tensors with guard bands of CANARY_BYTE before and after
    each one; check() asserts that no kernel wrote outside its output."""

    def __init__(self):
        self._bufs = []

    def empty(self, shape, dtype, device="cuda"):
        import torch
        n = int(np.prod(shape, dtype=np.int64)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((CANARY_BYTES + n + CANARY_BYTES,), CANARY_BYTE, dtype=torch.uint8,
                         device=device)
        self._bufs.append(buf)
        return buf[CANARY_BYTES:CANARY_BYTES + n].view(dtype).view(shape)

    def like(self, t):
        return self.empty(tuple(t.shape), t.dtype, t.device)

    def check(self):
        import torch
        torch.cuda.synchronize()
        for i, buf in enumerate(self._bufs):
            lo = buf[:CANARY_BYTES]
            hi = buf[-CANARY_BYTES:]
            assert bool((lo == CANARY_BYTE).all()), f"output {i}: guard band before it was written"
            assert bool((hi == CANARY_BYTE).all()), f"output {i}: guard band after it was written"


def topk_exact(gpu_ids: np.ndarray, ref_ids: np.ndarray, ref_logits: np.ndarray, s: int,
               gpu_logits=None, label: str = "") -> None:
    """Top-s ids must equal the oracle's exactly (the inputs are guarded so
    that the order is unique: tests/guards.py, G1).  When the GPU logits are
    given, print the largest GPU error beside the smallest top-(s+1) margin,
    both relative to the row's rms, to show the headroom."""
    from tests.guards import topk_margin
    np.testing.assert_array_equal(gpu_ids, ref_ids, err_msg=label)
    if gpu_logits is not None:
        B, K, _ = ref_logits.shape
        err = margin = 0.0
        margin = np.inf
        for b in range(B):
            for k in range(K):
                row = ref_logits[b, k]
                rms = float(np.sqrt(np.mean(row * row)))
                err = max(err, float(np.abs(gpu_logits[b, k] - row).max()) / rms)
                margin = min(margin, topk_margin(row, s + 1))
        print(f"{label}: top-s ids exact; max GPU logit error {err:.2e} rms, "
              f"smallest top-{s + 1} gap {margin:.2e} rms", flush=True)
