"""The forward pass captured in a HIP graph (torch.cuda.CUDAGraph on the
stream the library launches on) and replayed: every replay, with eager work
and synchronisations between replays, matches the eager call bit for bit
(needs an MI355X).  The library records no memset or allocation into the
graph: its kernels write every byte they later read."""
import numpy as np
import pytest

import workloads
from ssd_testlib import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw", [
    ("bf16_whole", dict(batch=2, seqlen=700, nheads=8, headdim=64, dstate=128, ngroups=1,
                        chunk_size=256, io="bf16")),
    ("bf16_split", dict(batch=1, seqlen=3000, nheads=4, headdim=64, dstate=64, ngroups=2,
                        chunk_size=128, io="bf16")),
    ("f32", dict(batch=2, seqlen=300, nheads=2, headdim=32, dstate=32, ngroups=1,
                 chunk_size=64, io="f32")),
])
def test_graph_replay_matches_eager(name, kw):
    import torch
    import ssd_chunked_scan_amd as ssd
    wl = workloads.custom_workload(name=f"graph_{name}", **kw)
    inp = workloads.make_inputs(wl, seed=31)
    t = to_device(inp)
    y_e, f_e = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None,
                           chunk_size=wl.chunk_size)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        launch, y, fs = ssd.prepare_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None,
                                        chunk_size=wl.chunk_size, stream=s.cuda_stream)
        launch()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        launch()
    for k in range(4):
        y.fill_(float("nan"))
        fs.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e) and torch.equal(fs, f_e), f"replay {k}"
        # eager work between replays
        y2, _ = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None,
                            chunk_size=wl.chunk_size)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_e)
