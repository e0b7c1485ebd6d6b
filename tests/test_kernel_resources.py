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

The heads' stage-2 index arithmetic is modelled too: the 8-row tile's
lane-to-(row, chunk) map, the LDS order of its B operand and the two-half
sum against direct dot products, and the XCD-weighted split of the tiles
over the workgroups with the inverse the merge kernel uses.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np
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


# ---------------------------------------------------------------------------
# The pipelined bf16 dh = 128 kernel: LDS layout of a stage and its schedule.

PIPE_RB, PIPE_OP = 256, 16384   # bytes per key row, bytes per operand and stage


def _pipe_stage_lds(Kst, Vst):
    """The K and V buffers (as 16-bit words) after every wave's direct loads
    of one 64-key stage: wave w, instruction i moves key rows 4 (w + 8 i) ..
    + 3, lane l landing at byte l * 16 of its kilobyte with chunk
    (l % 16) ^ swizzle(row) of row 4 (w + 8 i) + l / 16."""
    kl = np.full(PIPE_OP // 2, -1, np.int64)
    vl = np.full(PIPE_OP // 2, -1, np.int64)
    kg, vg = Kst.reshape(-1), Vst.reshape(-1)
    for wave in range(8):
        for lane in range(64):
            row0 = 4 * wave + (lane >> 4)
            cv = ((lane & 15) ^ (4 * (lane >> 4))) * 16
            for i, row in enumerate((row0, row0 + 32)):
                ok = row * PIPE_RB + ((lane & 15) ^ (row & 15)) * 16
                ov = row * PIPE_RB + cv
                dst = ((wave + 8 * i) * 1024 + lane * 16) // 2
                assert (kl[dst:dst + 8] == -1).all() and (vl[dst:dst + 8] == -1).all()
                kl[dst:dst + 8] = kg[ok // 2:ok // 2 + 8]
                vl[dst:dst + 8] = vg[ov // 2:ov // 2 + 8]
    return kl, vl


def test_pipelined_attention_lds_fragments():
    """Every lane's K fragment (ds_read_b128) and V^T fragment (two
    ds_read_b64_tr_b16: within 16 lanes, lane i receives element i of the
    four 8-byte rows addressed by lanes 4r + q) are the MFMA operands the
    kernel assumes; every read stays inside its 16 KiB buffer and hits
    distinct LDS banks per pass."""
    rng = np.random.default_rng(3)
    Kst = rng.integers(0, 1 << 16, size=(64, 128))
    Vst = rng.integers(0, 1 << 16, size=(64, 128))
    kl, vl = _pipe_stage_lds(Kst, Vst)
    assert (kl >= 0).all() and (vl >= 0).all()
    for sub in range(2):
        for ks in range(8):
            offs = []
            for lane in range(64):
                col, h = lane & 31, lane >> 5
                off = col * PIPE_RB + ((32 * ks) ^ (16 * (h ^ (col & 15)))) + sub * 8192
                assert off + 16 <= PIPE_OP
                got = kl[off // 2:off // 2 + 8]
                assert (got == Kst[32 * sub + col, 16 * ks + 8 * h:16 * ks + 8 * h + 8]).all()
                offs.append(off)
            for p in range(4):   # 16 lanes per pass, 16 distinct 16-byte bank groups
                assert len({(a // 16) % 16 for a in offs[16 * p:16 * p + 16]}) == 16
        for mm in range(2):
            for dt in range(4):
                A = np.zeros((64, 8), np.int64)
                for rd in range(2):
                    addr = []
                    for lane in range(64):
                        h, r4, q, gm = lane >> 5, (lane >> 2) & 3, lane & 3, (lane >> 4) & 1
                        va = (4 * h + r4) * PIPE_RB + (2 * gm + (q >> 1)) * 16 + (q & 1) * 8 + 64 * (dt ^ r4)
                        a = va + sub * 8192 + (16 * mm + 8 * rd) * PIPE_RB
                        assert a + 8 <= PIPE_OP
                        addr.append(a)
                    for g in range(4):
                        for i in range(16):
                            for r in range(4):
                                A[16 * g + i, 4 * rd + r] = vl[addr[16 * g + 4 * r + i // 4] // 2 + i % 4]
                    for p in range(2):   # 32 lanes of 8 bytes per pass: all 64 banks
                        banks = set()
                        for a in addr[32 * p:32 * p + 32]:
                            banks |= {(a // 4) % 64, (a // 4 + 1) % 64}
                        assert len(banks) == 64
                for lane in range(64):
                    h = lane >> 5
                    for e in range(8):
                        key = 32 * sub + 16 * mm + 4 * h + 8 * (e // 4) + e % 4
                        assert A[lane, e] == Vst[key, 32 * dt + (lane & 31)]
                        # the same key as element e of the P^T operand: score
                        # r = 8 mm + e of the lane (key 8 (r / 4) + 4 h + r % 4)
                        r = 8 * mm + e
                        assert key == 32 * sub + 8 * (r // 4) + 4 * h + r % 4


@pytest.mark.parametrize("nstage", [1, 2, 3, 4, 5, 8, 131])
def test_pipelined_attention_schedule(nstage):
    """Four stage buffers, loads three stages ahead, one barrier per stage.
    Before the first step stages 0-2 are issued, the wave waits for all but
    the latest stage and a barrier follows; then block 0 is read.  Step s
    issues stage s + 3 into buffer (s + 3) mod 4, reads stage s (buffer
    s mod 4) and the first half of stage s + 1 (buffer (s + 1) mod 4), waits
    for all but the latest stage's loads, barrier.  Every read must find its
    stage in the buffer and landed before the last barrier; a buffer is
    loaded again only after the last read of its previous stage, in an
    earlier barrier interval."""
    held = {}          # buffer -> stage it holds (or is receiving)
    issued = []        # stages in issue order
    landed = set()     # stages whose loads are complete
    visible = set()    # stages landed before the last barrier
    last_read = {}     # stage -> step of its last read (-1: before the first step)

    def issue(t, step):
        b = t % 4
        prev = held.get(b)
        if prev is not None:
            assert last_read.get(prev, -2) < step, (t, prev, step)
        held[b] = t
        issued.append(t)

    def read(t, step):
        assert held[t % 4] == t and t in visible, (t, step, held)
        last_read[t] = step

    for t in range(3):
        issue(t, -1)
    landed.update(issued[:-1])
    visible = set(landed)
    read(0, -1)
    for s in range(nstage):
        issue(s + 3, s)
        read(s, s)
        read(s + 1, s)    # past the last stage: a reload of the last one, its result unused
        landed.update(issued[:-1])
        visible = set(landed)


def test_no_bit_cast_of_vector_elements():
    """__builtin_bit_cast of an ext_vector element (v[i]) compiles to a cast
    of element 0 whatever i is (seen in the attention kernel's row sums);
    the sources must cast scalars instead."""
    bad = []
    for src in SOURCES + ["common.h"]:
        for n, line in enumerate(open(os.path.join(CSRC, src)), 1):
            if re.search(r"__builtin_bit_cast\([^,]+,\s*[\w.]+\[[^\]]+\]\s*\)", line):
                bad.append(f"{src}:{n}: {line.strip()}")
    assert not bad, bad


def _mfma16(a_lanes, b_lanes):
    """16x16 MFMA tile over one k-step as the hardware defines it: lane l
    brings row l % 16 of A and column l % 16 of B, its elements covering lane
    group l / 16's share of k; the result element r of lane l is
    C[4 (l / 16) + r][l % 16]."""
    C = np.zeros((16, 16))
    for i in range(16):
        for j in range(16):
            C[i, j] = sum(float(np.dot(a_lanes[16 * g + i], b_lanes[16 * g + j])) for g in range(4))
    return np.array([[C[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(64)])


@pytest.mark.parametrize("kc,B,cg", [(8, 1, 1), (8, 8, 1), (4, 5, 1), (8, 16, 2), (8, 9, 2), (4, 12, 2)])
def test_heads_rows8_layout(kc, B, cg):
    """The 8-row stage-2 tile: lane (c, g) loads W row c % 8 at chunk
    4 (c / 8) + g of each 128-byte step (kc elements per 16-byte chunk) and
    reads its B operand from LDS entry [slot][step][lane], filled with column
    8 slot + c % 8 (clamped to B - 1) of z at the same chunk; then for every
    live lane (g < 2, c < 8, column 8 q + c < B) acc + acc of lane + 40 is the
    dot product of tile row 4 g + r with that column over the whole row."""
    rng = np.random.default_rng(11)
    steps = 3
    d = steps * 8 * kc
    rows, tile = 21, 2                       # a ragged tile: rows 16..20 exist, 21..23 clamp
    W = rng.standard_normal((rows, d))
    z = rng.standard_normal((B, d))
    # the LDS fill: entry [slot][t][q]
    zl = np.zeros((cg, steps, 64, kc))
    for slot in range(cg):
        for t in range(steps):
            for q in range(64):
                cq = q % 16
                col = min((slot * 8 if cg == 2 else 0) + cq % 8, B - 1)
                off = t * 8 * kc + (cq // 8) * 4 * kc + (q // 16) * kc
                zl[slot, t, q] = z[col, off:off + kc]
    acc = np.zeros((cg, 64, 4))
    for t in range(steps):
        a_lanes = []
        for lane in range(64):
            c, g = lane % 16, lane // 16
            r = min(tile * 8 + c % 8, rows - 1)
            off = t * 8 * kc + (c // 8) * 4 * kc + g * kc
            a_lanes.append(W[r, off:off + kc])
        for q in range(cg):
            acc[q] += _mfma16(a_lanes, [zl[q, t, lane] for lane in range(64)])
    for q in range(cg):
        for lane in range(64):
            c, g = lane % 16, lane // 16
            col = q * 8 + c
            if not (g < 2 and c < 8 and col < B):
                continue
            for r in range(4):
                v = tile * 8 + 4 * g + r
                full = acc[q, lane, r] + acc[q, (lane + 40) % 64, r]
                if v < rows:
                    assert abs(full - float(np.dot(W[v], z[col]))) < 1e-9


# ------------------------------------------------- stage-2 workgroup split
# Mirrors of the device formulas in heads.hip (wg_tiles, tile_wg,
# head_wg_first / head_wg_count): the weighted split must cover every tile
# once, in order, leave no workgroup empty, keep a workgroup within two heads
# (its LDS holds two head slots), and the merge's inverse must name the owner
# of every tile.
XCD_SHARE = 32


def _share_prefix(j, base, wt):
    if not wt:
        return j
    return XCD_SHARE * j + ((-1 if base & 1 else 1) if j & 1 else 0)


XCD_MIN_TILES = 32   # per wave, four waves per workgroup


def _weighted(ntph, nt, P, G):
    return ntph >= XCD_MIN_TILES * 4 * G if G > 0 else nt >= XCD_MIN_TILES * 4 * P


def _wg_tiles(wg, ntph, nt, P, G):
    wt = _weighted(ntph, nt, P, G)
    if G > 0:
        h, j = wg // G, wg % G
        D = _share_prefix(G, h * G, wt)
        return (h * ntph + ntph * _share_prefix(j, h * G, wt) // D,
                h * ntph + ntph * _share_prefix(j + 1, h * G, wt) // D)
    D = _share_prefix(P, 0, wt)
    return nt * _share_prefix(wg, 0, wt) // D, nt * _share_prefix(wg + 1, 0, wt) // D


def _tile_wg(t, ntph, nt, P):
    if not _weighted(ntph, nt, P, 0):
        return ((t + 1) * P - 1) // nt
    D = _share_prefix(P, 0, True)
    X = ((t + 1) * D - 1) // nt
    w = X // XCD_SHARE
    if (w & 1) and X % XCD_SHARE == 0:
        w -= 1
    return min(w, P - 1)


@pytest.mark.parametrize("nh,ntph,cg", [(4, 4000, 1), (5, 16032, 1), (6, 16032, 1), (4, 125, 1),
                                        (3, 64, 1), (17, 13, 1), (1, 2, 1), (5, 513, 1), (1, 32768, 1),
                                        (2, 16385, 1), (16, 2049, 1), (1, 32769, 2),
                                        (4, 4000, 2), (5, 4000, 2), (3, 377, 2), (2, 13, 2),
                                        (17, 9000, 2), (1, 1, 2)])
def test_stage2_workgroup_split(nh, ntph, cg):
    nt = nh * ntph
    if cg == 2:
        G = max(1, min(256 // nh, ntph))
        P = G * nh
    else:
        G, P = 0, min(nt, 256)
    owner = {}
    prev_end = 0
    for wg in range(P):
        beg, end = _wg_tiles(wg, ntph, nt, P, G)
        if G > 0:
            h = wg // G
            assert beg >= h * ntph and end <= (h + 1) * ntph
        assert beg < end, (wg, beg, end)            # never empty
        if G == 0:
            assert beg == prev_end                   # in order, no gap
            assert (end - 1) // ntph - beg // ntph <= 1   # at most two heads
        prev_end = end
        for t in range(beg, end):
            assert t not in owner
            owner[t] = wg
    assert len(owner) == nt
    if G == 0:
        for t in range(nt):
            assert _tile_wg(t, ntph, nt, P) == owner[t]
        for h in range(nh):
            first = _tile_wg(h * ntph, ntph, nt, P)
            last = _tile_wg(h * ntph + ntph - 1, ntph, nt, P)
            assert {owner[t] for t in range(h * ntph, (h + 1) * ntph)} == set(range(first, last + 1))
    # the weighting: even hardware ids take 33 shares per 31 of odd ones
    if _weighted(ntph, nt, P, G) and G == 0 and P == 256:
        ev = sum(_wg_tiles(w, ntph, nt, P, G)[1] - _wg_tiles(w, ntph, nt, P, G)[0] for w in range(0, P, 2))
        od = nt - ev
        assert 1.03 < ev / od < 1.09   # 33/31 up to the rounding of whole tiles
