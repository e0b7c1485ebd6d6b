"""CPU: register and scratch budgets of the gfx950 kernels, and the K/V
staging schedule of the tree-attention kernel.

Every kernel must run from registers alone: no vector register spilled to
scratch memory and no private (scratch) segment.  The tree-attention kernel
runs two waves per SIMD, so it has 256 registers per lane; with a deeper
load prefetch (three or four register sets of staged K/V) the compiler
spills staging registers to scratch, the one structural difference between
the prefetch depth that shipped and the depth that was dropped.

The staging schedule (which register set holds which stage, which LDS
buffer each stage is written to and read from, and when) is modelled step
by step for prefetch depths 1 to 4: every stage computed must be the one
its buffer holds, and no buffer may be overwritten before the barrier that
follows its last read.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "medusa_tree_verification_amd", "csrc")
SOURCES = ["heads.hip", "tree_attention.hip", "tree_accept.hip", "tree_commit.hip", "forward.hip",
           "probes.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _kernels(asm: str):
    meta = asm[asm.index("amdhsa.kernels:"):]
    out = []
    for blk in re.split(r"\n  - ", meta)[1:]:
        d = {}
        for key in (".name", ".vgpr_spill_count", ".private_segment_fixed_size", ".vgpr_count"):
            m = re.search(r"\n\s+" + re.escape(key) + r":\s+(\S+)", "\n" + blk)
            if m:
                d[key] = m.group(1)
        if ".name" in d:
            out.append(d)
    return out


def _device_asm(src, tmp):
    out = os.path.join(tmp, src + ".s")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                           "--cuda-device-only", "-S", "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           "-o", out, os.path.join(CSRC, src)], stderr=subprocess.DEVNULL,
                          timeout=1800)
    return open(out).read()


@pytest.fixture(scope="module")
def asms(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    tmp = str(tmp_path_factory.mktemp("asm"))
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        return dict(zip(SOURCES, ex.map(lambda s: _device_asm(s, tmp), SOURCES)))


def _function(asm: str, name: str) -> str:
    start = asm.index("\n" + name + ":")
    return asm[start:asm.index(".Lfunc_end", start)]


def test_no_kernel_spills_to_scratch(asms):
    seen = 0
    for src, asm in asms.items():
        for k in _kernels(asm):
            seen += 1
            assert k.get(".vgpr_spill_count", "0") == "0", (src, k)
            assert k.get(".private_segment_fixed_size", "0") == "0", (src, k)
            assert int(k[".vgpr_count"]) <= 512, (src, k)
    assert seen >= 40


def _model_ring(PD, nstage):
    """The eight-wave kernel's schedule: PD register sets, two LDS buffers,
    one barrier per stage.  Within one barrier interval the waves run in any
    order, so no buffer may be both written and read in the same interval.
    Returns the (stage computed, stage its buffer holds) pairs."""
    held = {k: k for k in range(PD)}   # register set -> stage whose loads it holds
    lds = {0: None, 1: None}
    # prologue interval: stage 0 stored, its set re-issued with stage PD
    lds[0] = held[0]
    held[0] = PD
    computed = []
    nstage_pad = (nstage + PD - 1) // PD * PD
    for base in range(0, nstage_pad, PD):
        for k in range(PD):
            sidx = base + k
            reg = (k + 1) % PD             # the set holding stage sidx + 1
            wbuf = (sidx + 1) & 1
            assert held[reg] == sidx + 1, (PD, sidx, held)
            lds[wbuf] = held[reg]
            held[reg] = sidx + 1 + PD
            reads = set()
            if sidx < nstage:
                rbuf = sidx & 1
                computed.append((sidx, lds[rbuf]))
                reads.add(rbuf)
            assert wbuf not in reads, (PD, sidx, "buffer written and read in one interval")
    return computed


@pytest.mark.parametrize("PD", [1, 2, 3, 4])
@pytest.mark.parametrize("nstage", [1, 2, 3, 5, 8, 129])
def test_attention_staging_schedule(PD, nstage):
    computed = _model_ring(PD, nstage)
    assert [s for s, _ in computed] == list(range(nstage))
    assert all(s == held for s, held in computed)


def test_shipped_prefetch_depth_is_two():
    src = open(os.path.join(CSRC, "tree_attention.hip")).read()
    assert re.search(r"constexpr int kPD = 2;", src)


def test_big_gemm_waits_only_on_its_stage_loads(asms):
    """gemm_big_kernel waits on the vector-memory counter with fixed
    immediates (all of this wave's loads, or all but the 16 of one stage)
    and crosses its barriers without fences; that is right only while the
    stage loads are the wave's only vector-memory operations in flight.  So
    up to its last barrier the kernel may issue no other vector-memory
    instruction than the direct-to-LDS stage loads."""
    body = _function(asms["forward.hip"], "_ZN6medusa12_GLOBAL__N_115gemm_big_kernelENS0_8GemmArgsE")
    last_barrier = body.rindex("s_barrier")
    vmem = re.findall(r"^\s+((?:global|buffer|flat|scratch)_\w+)", body[:last_barrier], re.M)
    assert vmem and set(vmem) == {"global_load_lds_dwordx4"}, sorted(set(vmem))
    assert "s_waitcnt vmcnt(16)" in body and "s_waitcnt vmcnt(0)" in body
