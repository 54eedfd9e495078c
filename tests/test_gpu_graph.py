"""rr_prefill captured in a HIP graph and replayed.

The library enqueues only kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a caller may capture a whole prefill step
into a graph.  Each replay must give bitwise the eager result.  Between the
replays the inputs are overwritten and restored by eager work, so a replay
that reused stale state would show.
"""
import numpy as np
import pytest
import torch

from tests.helpers import small_workload

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("shape", [
    ("llama", 1216, 8, 2, 128, 128, 8, 0.9),
    ("video", 2048, 7, 1, 128, 128, 16, 0.95),
], ids=str)
def test_prefill_graph_replays_match_eager(shape):
    import long_context_prefill_rr_amd as rr
    kind, L, Hq, Hkv, d, B, S, tau = shape
    print("graph %s" % (shape,), flush=True)
    w, g = small_workload(kind=kind, L=L, Hq=Hq, Hkv=Hkv, d=d, B=B, S=S, seed=17)
    q, k, v = _dev(g["q"]), _dev(g["k"]), _dev(g["v"])
    nb = -(-L // B)
    O = torch.empty((L, Hq, d), dtype=torch.float32, device="cuda")
    counts = torch.empty((Hq, nb), dtype=torch.int32, device="cuda")
    idx = torch.empty((Hq, nb, nb), dtype=torch.int32, device="cuda")
    ws = torch.empty(rr.prefill_workspace_bytes(L, Hq, Hkv, d, B, S), dtype=torch.uint8, device="cuda")

    rr.rr_prefill(q, k, v, B, S, tau, out=O, counts=counts, block_idx=idx, ws=ws)
    torch.cuda.synchronize()
    O_ref, c_ref, i_ref = O.clone(), counts.clone(), idx.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rr.rr_prefill(q, k, v, B, S, tau, out=O, counts=counts, block_idx=idx, ws=ws)  # warm on the side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rr.rr_prefill(q, k, v, B, S, tau, out=O, counts=counts, block_idx=idx, ws=ws)
    torch.cuda.synchronize()

    q_saved = q.clone()
    for r in range(3):
        # Eager work between replays: scribble over the outputs and the
        # workspace, and perturb then restore q.
        O.fill_(float("nan"))
        counts.fill_(-7)
        idx.fill_(-7)
        ws.fill_(0xA5)
        q.mul_(2)
        q.copy_(q_saved)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(counts, c_ref), r
        assert torch.equal(idx, i_ref), r
        assert torch.equal(O, O_ref), r
    print("  3 replays bitwise equal to the eager run", flush=True)
