"""The benchmark step (spicy_coarsen of the per-step chunk, then the
shared-prefix decode) captured as one HIP graph and replayed: every replay
gives the eagerly issued step's results bit for bit (cache pools, lengths,
O and LSE).  Before each replay the outputs and the step's lengths are
overwritten, so that a replay that wrote nothing would show; between replays
the program runs its own eager step and synchronises.  The captured calls
allocate nothing and record no memset (the library has neither)."""
import numpy as np
import pytest
import torch

from coarse_grained_decode_amd import workloads as W
from test_gpu_parity import DEV, _need_gpu, host

pytestmark = pytest.mark.gpu


def snapshot(dw):
    c = dw.cache
    return dict(k=host(c.k).copy(), v=host(c.v).copy(), ab=host(c.ab).copy(), meta=host(c.meta).copy(),
                lengths=dw.step.lengths.cpu().numpy(), o=dw.o.cpu().numpy(), lse=dw.lse.cpu().numpy())


def test_captured_step_replays_equal_the_eager_step():
    import coarse_grained_decode_amd as cgd
    from coarse_grained_decode_amd.runner import DeviceWorkload
    _need_gpu()
    wl = W.shared_prefix(B=5, prefix_T=6000, chunk_T=2000, suffix_range=(100, 400))
    print(f"[graph] {wl.name}: B={wl.B} pages={wl.num_pages}", flush=True)
    dw = DeviceWorkload.of(wl, DEV, meta=True, fill=float("nan"))
    dw.run_setup()
    dw.step_once()
    torch.cuda.synchronize()
    want = snapshot(dw)
    assert int(dw.step.ws[0].item()) == 0 and cgd.device_error(dw.dws) == 0
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dw.step_once()
    torch.cuda.synchronize()
    for r in range(3):
        dw.o.fill_(float("nan"))
        dw.lse.fill_(float("nan"))
        dw.step.lengths.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(dw)
        for name in want:
            assert got[name].tobytes() == want[name].tobytes(), f"replay {r}: {name} differs"
        assert int(dw.step.ws[0].item()) == 0 and cgd.device_error(dw.dws) == 0
        dw.step_once()                      # the program's own eager work between replays
        torch.cuda.synchronize()
