"""The C-ABI library: exported symbols, workspace sizing and host-side
argument validation (CPU only: every call here fails validation before any
GPU work is enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "medusa_verify.h")


PROBE_HEADER = os.path.join(ROOT, "include", "medusa_probes.h")


def _declared(header=HEADER):
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", txt)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def mv():
    """The binding; MEDUSA_VERIFY_TEST_LIB names another build of the same
    sources to check instead (the sanitizer build of test_sanitizers.py)."""
    from medusa_tree_verification_amd import binding
    path = os.environ.get("MEDUSA_VERIFY_TEST_LIB")
    if path:
        saved = binding.lib
        binding.lib = binding._load(path)
        yield binding
        binding.lib = saved
    else:
        yield binding


def test_every_declared_symbol_is_exported(mv):
    names = _declared()
    assert "medusa_heads_topk" in names and "tree_attention" in names and "tree_accept" in names
    for n in names:
        assert hasattr(mv.lib, n), n
    assert set(names) == set(mv.EXPORTS)
    probes = _declared(PROBE_HEADER)
    assert set(probes) == set(mv.PROBE_EXPORTS)
    for n in probes:
        assert hasattr(mv.lib, n), n


def test_probe_validation(mv):
    L = mv.lib
    # one word per thread: the read probe's 256 x 256 threads, the MFMA probe's 256 x 4 waves
    assert L.medusa_probe_sink_bytes() >= max(256 * 256, 256 * 4 * 64) * 4
    assert L.medusa_probe_read(None, 16, FAKE, None) == -1
    assert L.medusa_probe_read(FAKE, 15, FAKE, None) == -2
    assert L.medusa_probe_read(ctypes.c_void_p(0x1008), 16, FAKE, None) == -2
    assert L.medusa_probe_mfma(0, FAKE, None) == -6
    assert L.medusa_probe_read_timed(FAKE, 16, FAKE, None, 0, None) == -1
    assert L.medusa_probe_read_timed(FAKE, 15, FAKE, FAKE, 0, None) == -2
    assert L.medusa_probe_read_timed(FAKE, 16, FAKE, FAKE, 2, None) == -6
    assert L.medusa_probe_read_timed(FAKE, 4096, FAKE, FAKE, 1, None) == -2
    assert L.medusa_probe_read_workgroups() == 256
    assert L.medusa_probe_mfma(1, None, None) == -1
    assert L.medusa_probe_mfma_flops(10) == 256 * 4 * 8 * 10 * 32 * 32 * 16 * 2


def test_status_strings_and_version(mv):
    assert mv.lib.medusa_abi_version() == 1
    for code in range(-8, 1):
        assert mv.status_str(code) and mv.status_str(code) != "unknown status"
    assert mv.status_str(5) == "unknown status"


def test_workspace_sizes(mv):
    L = mv.lib
    assert L.medusa_heads_topk_workspace_bytes(1, 4, 4096, 32000, 3, 1) >= 4 * 4096 * 2
    assert L.medusa_heads_topk_workspace_bytes(17, 4, 4096, 32000, 3, 1) == 0     # B > 16
    assert L.medusa_heads_topk_workspace_bytes(1, 4, 4000, 32000, 3, 1) == 0      # d % 128
    assert L.medusa_heads_topk_workspace_bytes(1, 4, 4096, 2, 3, 1) == 0          # s > V
    assert L.tree_attention_workspace_bytes(1, 32, 32, 2048, 128, 64, 1) > 0
    assert L.tree_attention_workspace_bytes(1, 32, 5, 2048, 128, 64, 1) == 0      # Hq % Hkv
    assert L.tree_attention_workspace_bytes(1, 32, 8, 2048, 96, 64, 1) == 0       # dh
    assert L.tree_attention_workspace_bytes(1, 32, 8, 2048, 128, 257, 1) == 0     # T
    assert L.tree_accept_workspace_bytes(8, 256, 128256, 5, 3) >= 8 * 256


FAKE = ctypes.c_void_p(0x1000)       # never dereferenced: validation fails first
FAKE_WS = ctypes.c_void_p(0x10000)   # 256-aligned


def _i32(xs):
    arr = (ctypes.c_int32 * len(xs))(*xs)
    return arr


def test_heads_validation(mv):
    L = mv.lib
    ok = dict(B=1, K=4, d=4096, V=32000, s=3, dt=1)

    def call(hidden=FAKE, w1=FAKE, w2=FAKE, ids=FAKE, ws=FAKE_WS, wsb=1 << 40, **kw):
        a = dict(ok, **kw)
        return L.medusa_heads_topk(hidden, w1, w2, a["B"], a["K"], a["d"], a["V"], a["s"], a["dt"],
                                   None, ids, None, ws, wsb, None)
    assert call(hidden=None) == -1
    assert call(w1=None) == -1
    assert call(ids=None) == -1
    assert call(dt=7) == -3
    assert call(B=0) == -2 and call(B=17) == -2 and call(d=100) == -2 and call(s=9) == -2
    assert call(K=0) == -2 and call(V=2) == -2
    assert call(ws=None) == -5
    assert call(ws=ctypes.c_void_p(0x10010)) == -5
    assert call(wsb=10) == -5
    assert L.medusa_heads_stage1(FAKE, None, 1, 4, 4096, 32000, 3, 1, FAKE_WS, 1 << 40, None) == -1
    assert L.medusa_heads_stage2(FAKE, 1, 4, 4096, 32000, 3, 1, None, None, None, FAKE_WS,
                                 1 << 40, None) == -1


def test_attention_validation(mv):
    L = mv.lib
    par = _i32([-1, 0, 0, 1])

    def call(parent=par, T=4, Hq=4, Hkv=2, dh=128, scale=0.1, dt=1, out=FAKE, ws=FAKE_WS,
             wsb=1 << 40, q=FAKE):
        return L.tree_attention(q, FAKE, FAKE, FAKE, FAKE, FAKE, parent, 2, Hq, Hkv, 64, dh, T,
                                scale, dt, out, None, ws, wsb, None)
    assert call(q=None) == -1 and call(out=None) == -1 and call(parent=None) == -1
    assert call(Hkv=3) == -2 and call(dh=96) == -2 and call(T=0) == -2 and call(T=300) == -2
    assert call(dt=2) == -3
    assert call(scale=0.0) == -6 and call(scale=float("nan")) == -6
    assert call(parent=_i32([0, 0, 0, 1])) == -4          # root not -1
    assert call(parent=_i32([-1, 0, 3, 1])) == -4         # parent after child
    assert call(ws=None) == -5 and call(wsb=0) == -5
    # grids past the launch limits and query blocks past one buffer resource
    big = dict(Hq=1 << 16, Hkv=1 << 16)
    assert L.tree_attention(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, par, 1 << 16, big["Hq"],
                            big["Hkv"], 0, 128, 4, 0.1, 1, FAKE, None, FAKE_WS, 1 << 40,
                            None) == -2
    assert L.tree_attention_workspace_bytes(1 << 16, 1 << 16, 1 << 16, 0, 128, 4, 1) == 0
    assert call(Hq=1 << 22, Hkv=1) == -2
    assert L.tree_attention_workspace_bytes(1, 1 << 22, 1, 64, 128, 4, 1) == 0


def test_accept_validation(mv):
    L = mv.lib
    par = _i32([-1, 0, 0, 1])

    def call(parent=par, rank=None, T=4, K=2, s=2, mode=0, temp=1.0, eps=0.09, delta=0.6, dt=1,
             ws=FAKE_WS, wsb=1 << 40, logits=FAKE):
        return L.tree_accept(logits, FAKE, parent, rank, 2, T, 100, K, s, dt, mode, temp, eps,
                             delta, FAKE, FAKE, FAKE, None, None, ws, wsb, None)
    assert call(logits=None) == -1 and call(parent=None) == -1
    assert call(dt=3) == -3
    assert call(mode=3) == -6 and call(mode=-1) == -6
    assert call(mode=2, temp=0.0) == -6 and call(mode=2, wsb=0) == -5
    assert call(mode=1, temp=0.0) == -6 and call(mode=1, eps=0.0) == -6
    assert call(mode=1, delta=-1.0) == -6
    assert call(mode=0, temp=0.0, wsb=0) == -5               # greedy ignores temperature
    assert call(K=1) == -4                                    # depth 2 > K
    assert call(s=1) == -4                                    # second child has rank 1
    assert call(rank=_i32([0, 1, 1, 0])) == -4                # siblings share a rank
    assert call(rank=_i32([0, 0, 5, 0])) == -4                # rank >= s
    assert call(T=257) == -2
    assert call(ws=None) == -5 and call(wsb=0) == -5


def test_commit_validation(mv):
    L = mv.lib
    par = _i32([-1, 0, 0, 1])

    def call(kc=FAKE, parent=par, B=2, Hkv=2, Lcap=64, dh=128, T=4, dt=1):
        return L.tree_commit_kv(kc, FAKE, FAKE, FAKE, FAKE, FAKE, parent, B, Hkv, Lcap, dh, T, dt,
                                None, None)
    assert call(kc=None) == -1 and call(parent=None) == -1
    assert call(dt=2) == -3
    assert call(B=0) == -2 and call(Hkv=0) == -2 and call(Lcap=-1) == -2
    assert call(dh=12) == -2                                  # 24 bytes: not a 16-byte multiple
    assert call(dt=0, dh=6) == -2 and call(T=0) == -2 and call(T=257) == -2
    assert call(parent=_i32([0, 0, 0, 1])) == -4              # root must be -1
    assert call(parent=_i32([-1, 0, 2, 1])) == -4             # parent[n] < n


def test_sample_validation(mv):
    L = mv.lib

    def call(logits=FAKE, rows=FAKE, u=FAKE, B=2, T=4, V=100, dt=1, temp=1.0, tok=FAKE):
        return L.medusa_sample_token(logits, rows, u, B, T, V, dt, temp, tok, None)
    assert call(logits=None) == -1 and call(rows=None) == -1 and call(u=None) == -1
    assert call(tok=None) == -1
    assert call(dt=2) == -3
    assert call(B=0) == -2 and call(T=0) == -2 and call(V=0) == -2
    assert call(temp=0.0) == -6 and call(temp=-1.0) == -6 and call(temp=float("inf")) == -6


def test_forward_validation(mv):
    L = mv.lib
    ok = dict(N=2, B=1, T=4, d=256, Hq=4, Hkv=2, dh=64, Lcap=128, V=1000, dt=1)
    par = _i32([-1, 0, 0, 1])
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    holes = (ctypes.c_void_p * 2)(0x1000, None)

    def call(h0=FAKE, g=ptrs, wq=ptrs, kc=ptrs, parent=par, logits=FAKE, ws=FAKE_WS, wsb=1 << 40,
             theta=10000.0, eps=1e-6, **kw):
        a = dict(ok, **kw)
        return L.medusa_verify_forward(h0, a["N"], g, wq, ptrs, ptrs, ptrs, FAKE, FAKE, kc, ptrs,
                                       FAKE, parent, a["B"], a["T"], a["d"], a["Hq"], a["Hkv"],
                                       a["dh"], a["Lcap"], a["V"], a["dt"], theta, eps, logits,
                                       None, None, None, ws, wsb, None)
    assert call(h0=None) == -1 and call(logits=None) == -1
    assert call(g=None) == -1 and call(wq=holes) == -1 and call(kc=holes) == -1
    assert call(dt=5) == -3
    assert call(N=-1) == -2 and call(N=257) == -2 and call(B=0) == -2 and call(T=257) == -2
    assert call(d=100) == -2 and call(d=16) == -2 and call(dh=96) == -2 and call(Hkv=3) == -2
    assert call(V=0) == -2 and call(B=64, T=256, V=200000) == -2
    assert call(dt=0, d=16, wsb=64) == -5       # fp32 takes d % 16 == 0 (fails later, on ws)
    assert call(theta=0.0) == -6 and call(theta=float("inf")) == -6 and call(eps=-1.0) == -6
    assert call(parent=_i32([0, 0, 0, 1])) == -4 and call(parent=_i32([-1, 0, 2, 1])) == -4
    assert call(ws=None) == -5 and call(ws=ctypes.c_void_p(0x10010)) == -5 and call(wsb=64) == -5
    # zero blocks: only the final norm and the LM head; the block arrays may be NULL
    assert call(N=0, g=None, wq=None, kc=None, ws=None) == -5
    ws = L.medusa_verify_forward_workspace_bytes(1, 4, 256, 4, 2, 64, 128, 1000, 1)
    assert ws >= 4 * 256 * 4                     # the fp32 residual stream at least
    assert L.medusa_verify_forward_workspace_bytes(1, 4, 100, 4, 2, 64, 128, 1000, 1) == 0


def test_stage2_split_validation(mv):
    L = mv.lib
    assert L.medusa_heads_stage2_stream(None, 1, 4, 4096, 32000, 3, 1, None, FAKE_WS, 1 << 40, None) == -1
    assert L.medusa_heads_stage2_stream(FAKE, 17, 4, 4096, 32000, 3, 1, None, FAKE_WS, 1 << 40, None) == -2
    assert L.medusa_heads_stage2_stream(FAKE, 1, 4, 4096, 32000, 3, 1, None, FAKE_WS, 64, None) == -5
    assert L.medusa_heads_stage2_merge(1, 4, 4096, 32000, 3, 1, None, None, FAKE_WS, 1 << 40, None) == -1
    assert L.medusa_heads_stage2_merge(1, 4, 4096, 32000, 9, 1, FAKE, None, FAKE_WS, 1 << 40, None) == -2
    assert L.medusa_heads_stage2_merge(1, 4, 4096, 32000, 3, 7, FAKE, None, FAKE_WS, 1 << 40, None) == -3
    assert L.medusa_heads_stage2_merge(1, 4, 4096, 32000, 3, 1, FAKE, None, None, 1 << 40, None) == -5


def test_bench_refuses_several_gpus():
    """The benchmark runs on one GPU; asking for more exits with a message
    before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_heads_noalloc_validation(mv):
    """The no-allocation heads call checks its arguments like medusa_heads_topk
    and rejects problems larger than its static scratch, all on the host."""
    L = mv.lib
    cap = L.medusa_heads_topk_noalloc_max_scratch()
    assert cap == 8 << 20

    def call(hidden=FAKE, w1=FAKE, w2=FAKE, ids=FAKE, B=1, K=4, d=4096, V=32000, s=3, dt=1):
        return L.medusa_heads_topk_noalloc(hidden, w1, w2, B, K, d, V, s, dt, None, ids, None,
                                           None)
    assert call(hidden=None) == -1 and call(ids=None) == -1
    assert call(dt=5) == -3 and call(B=17) == -2 and call(s=9) == -2
    # fp32, 16 sequences, 16 heads of 16384: z alone is 16 MiB
    assert L.medusa_heads_topk_workspace_bytes(16, 16, 16384, 1000, 3, 0) > cap
    assert call(B=16, K=16, d=16384, V=1000, dt=0) == -8
    assert "scratch" in mv.status_str(-8)
    # the largest workload's heads fit
    assert L.medusa_heads_topk_workspace_bytes(8, 5, 4096, 128256, 3, 1) <= cap
