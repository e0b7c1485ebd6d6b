"""GPU: the timed read probe records a start and an end for every workgroup."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pattern", [0, 1])
def test_probe_read_timed_stamps(pattern):
    import torch
    from medusa_tree_verification_amd import binding as mv
    dev = torch.device("cuda:0")
    sink = torch.empty(mv.lib.medusa_probe_sink_bytes() // 4, dtype=torch.int32, device=dev)
    buf = torch.ones(64 << 18, dtype=torch.int32, device=dev)   # 64 MiB
    nwg = mv.lib.medusa_probe_read_workgroups()
    stamps = torch.zeros(2 * nwg, dtype=torch.int32, device=dev)
    mv.probe_read_timed(buf, sink, stamps, pattern)
    torch.cuda.synchronize()
    st = stamps.cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    dur = (st[1::2] - st[0::2]) % (1 << 32)
    mhz = mv.lib.medusa_probe_clock_mhz()
    assert mhz > 0
    assert (dur > 0).all() and (dur / mhz < 1e6).all()   # every workgroup wrote, under a second
    # every 16-byte word of the all-ones buffer folds to 0 or 1 in each thread
    s = sink[: nwg * 256].cpu().numpy()
    assert set(np.unique(s)) <= {0, 1}
