"""rr_prefill_noalloc (the entry point that allocates nothing: its workspace
is a device array the library owns) against rr_prefill, through the C ABI.

Two calls in a row, the second on a smaller input, each compared with
rr_prefill on the same input: the same kernels run on the same inputs, so
the masks and outputs must be identical (this also shows the second call
does not depend on what the first left in the shared array).  A shape whose
workspace exceeds the array is refused before any launch.
"""
import numpy as np
import pytest
import torch

from tests.helpers import small_workload

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


CASES = [
    # (kind, L, Hq, Hkv, d, B, S, tau, out dtype): the 8K Llama shape, then a
    # smaller ragged G = 7 video-like shape with another d, B and S.
    ("llama", 8192, 32, 8, 128, 128, 8, 0.9, torch.float32),
    ("video", 1216, 7, 1, 64, 64, 16, 0.8, torch.bfloat16),
]


def _run_pair(case):
    import long_context_prefill_rr_amd as rr
    kind, L, Hq, Hkv, d, B, S, tau, odt = case
    w, g = small_workload(kind=kind, L=L, Hq=Hq, Hkv=Hkv, d=d, B=B, S=S, seed=23)
    q, k, v = _dev(g["q"]), _dev(g["k"]), _dev(g["v"])
    nb = w.nb
    print("noalloc case %s" % (case,), flush=True)
    O_ref, c_ref, i_ref = rr.rr_prefill(q, k, v, B, S, tau, out_dtype=odt)
    O = torch.full((L, Hq, d), float("nan"), dtype=odt, device="cuda")
    counts = torch.full((Hq, nb), -7, dtype=torch.int32, device="cuda")
    idx = torch.full((Hq, nb, nb), -7, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    rr.rr_prefill_noalloc(q, k, v, B, S, tau, out=O, counts=counts, block_idx=idx)
    torch.cuda.synchronize()
    assert torch.equal(counts, c_ref)
    assert torch.equal(idx, i_ref)
    assert torch.equal(O.view(torch.int16 if odt == torch.bfloat16 else torch.int32),
                       O_ref.view(torch.int16 if odt == torch.bfloat16 else torch.int32))


def test_noalloc_matches_prefill_twice_second_smaller():
    import long_context_prefill_rr_amd as rr
    assert rr.noalloc_scratch_bytes() == 64 << 20
    for case in CASES:
        kind, L, Hq, Hkv, d, B, S = case[:7]
        assert rr.prefill_workspace_bytes(L, Hq, Hkv, d, B, S) <= rr.noalloc_scratch_bytes()
        _run_pair(case)


def test_noalloc_refuses_shapes_beyond_its_array():
    import long_context_prefill_rr_amd as rr
    L, Hq, Hkv, d, B, S = 32768, 32, 8, 128, 128, 8
    assert rr.prefill_workspace_bytes(L, Hq, Hkv, d, B, S) > rr.noalloc_scratch_bytes()
    q = torch.zeros((L, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((L, Hkv, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rr.RRError) as e:
        rr.rr_prefill_noalloc(q, k, k, B, S, 0.9)
    assert e.value.code == 4   # RR_E_WORKSPACE
