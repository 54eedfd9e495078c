"""The C-ABI library loads, exports every symbol include/rr.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rr.h")
LIB = os.path.join(ROOT, "long_context_prefill_rr_amd", "librr.so")

RR_OK, RR_E_NULL, RR_E_SHAPE, RR_E_TAU, RR_E_WORKSPACE, RR_E_UNSUPPORTED = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rr_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from long_context_prefill_rr_amd import build
        build.build()
    from long_context_prefill_rr_amd import rr
    return rr.load_library()


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("rr_estimate", "rr_select", "rr_sparse_attn", "rr_prefill", "rr_mask_quality",
              "rr_xattn_estimate", "rr_rescue_estimate", "rr_merge_masks", "rr_estimate_materialized"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(lib, n)


def test_status_strings(lib):
    for c in range(7):
        assert lib.rr_status_str(c)
    assert lib.rr_abi_version() == 1


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _est(lib, L=1024, Hq=8, Hkv=2, d=128, B=128, S=8, ws_bytes=1 << 40, Q=FAKE):
    return lib.rr_estimate(Q, FAKE, L, Hq, Hkv, d, B, S, FAKE, FAKE, ws_bytes, None)


def test_estimate_validation(lib):
    assert _est(lib, Q=None) == RR_E_NULL
    assert _est(lib, L=1004) == RR_E_SHAPE           # L % S
    assert _est(lib, L=0) == RR_E_SHAPE
    assert _est(lib, Hq=6, Hkv=4) == RR_E_SHAPE      # Hq % Hkv
    assert _est(lib, S=256) == RR_E_SHAPE            # S > B
    assert _est(lib, S=12) == RR_E_SHAPE             # B % S
    assert _est(lib, d=96) == RR_E_UNSUPPORTED
    assert _est(lib, B=256, S=8) == RR_E_UNSUPPORTED
    assert _est(lib, ws_bytes=16) == RR_E_WORKSPACE
    assert _est(lib, L=128 * 4097) == RR_E_UNSUPPORTED
    assert _est(lib, Hq=2048, Hkv=2) == RR_E_UNSUPPORTED   # more than 1024 query heads
    assert lib.rr_select(FAKE, 2048, 1024, 128, ctypes.c_float(0.9), FAKE, FAKE, None) == RR_E_UNSUPPORTED


def test_workspace_sizes(lib):
    assert lib.rr_estimate_workspace_bytes(1004, 8, 2, 128, 128, 8) == 0
    a = lib.rr_estimate_workspace_bytes(8192, 32, 8, 128, 128, 8)
    b = lib.rr_sparse_attn_workspace_bytes(8192, 32, 8, 128, 128)
    c = lib.rr_prefill_workspace_bytes(8192, 32, 8, 128, 128, 8)
    assert a > 0 and b > 0 and c >= max(a, b) + 32 * 64 * 64 * 4
    # pooled-key planes + packed (row, block) pairs + row pairs
    ns, nb, c16 = 1024, 64, 16
    P = c16 * nb * (nb + 1) // 2
    assert a >= 3 * 8 * ns * 128 * 2 + 32 * P * 8 + 32 * ns * 8


def test_one_workspace_size_serves_every_call(lib):
    # rr_workspace_bytes(L, Hq, Hkv, d, B, S): the largest workspace any call
    # needs on the shape, so one buffer of that size serves them all.
    for L, Hq, Hkv, d, B, S in [(8192, 32, 8, 128, 128, 8), (1216, 7, 1, 64, 64, 16),
                                (131072, 32, 8, 128, 128, 8), (1024, 8, 8, 64, 128, 1),
                                (65536, 28, 4, 128, 128, 16)]:
        w = lib.rr_workspace_bytes(L, Hq, Hkv, d, B, S)
        per_call = [lib.rr_estimate_workspace_bytes(L, Hq, Hkv, d, B, S),
                    lib.rr_sparse_attn_workspace_bytes(L, Hq, Hkv, d, B),
                    lib.rr_prefill_workspace_bytes(L, Hq, Hkv, d, B, S),
                    lib.rr_rescue_workspace_bytes(L, Hq, Hkv, d, B),
                    lib.rr_estimate_materialized_workspace_bytes(L, Hq, Hkv, d, B, S)]
        assert w > 0 and w == max(per_call), (L, Hq, Hkv, d, B, S, w, per_call)
    # Invalid or unsupported shapes give 0, as the calls reject them.
    assert lib.rr_workspace_bytes(1004, 8, 2, 128, 128, 8) == 0      # L % S
    assert lib.rr_workspace_bytes(1024, 6, 4, 128, 128, 8) == 0      # Hq % Hkv
    assert lib.rr_workspace_bytes(1024, 8, 2, 96, 128, 8) == 0       # d
    assert lib.rr_workspace_bytes(1024, 8, 2, 128, 128, 12) == 0     # B % S


def test_noalloc_prefill_validation(lib):
    # Host-side checks run before any HIP call: the rr_prefill rules, then the
    # size of the library-owned workspace.
    assert lib.rr_noalloc_scratch_bytes() == 64 << 20
    f = ctypes.c_float
    def p(L=1024, Hq=8, Hkv=2, d=128, B=128, S=8, tau=0.9, Q=FAKE, o_dtype=0):
        return lib.rr_prefill_noalloc(Q, FAKE, FAKE, L, Hq, Hkv, d, B, S, f(tau), FAKE, o_dtype,
                                      FAKE, FAKE, None)
    assert p(Q=None) == RR_E_NULL
    assert p(L=1004) == RR_E_SHAPE
    assert p(tau=0.0) == RR_E_TAU
    assert p(d=96) == RR_E_UNSUPPORTED
    assert p(o_dtype=5) == RR_E_UNSUPPORTED
    # 32K at 32/8 heads needs more than the 64 MiB array; 16K fits.
    assert lib.rr_prefill_workspace_bytes(16384, 32, 8, 128, 128, 8) <= 64 << 20
    assert lib.rr_prefill_workspace_bytes(32768, 32, 8, 128, 128, 8) > 64 << 20
    assert p(L=32768, Hq=32, Hkv=8) == RR_E_WORKSPACE


def test_select_and_attn_validation(lib):
    f = ctypes.c_float
    assert lib.rr_select(FAKE, 8, 1024, 128, f(0.0), FAKE, FAKE, None) == RR_E_TAU
    assert lib.rr_select(FAKE, 8, 1024, 128, f(1.5), FAKE, FAKE, None) == RR_E_TAU
    assert lib.rr_select(FAKE, 8, 1024, 128, f(float("nan")), FAKE, FAKE, None) == RR_E_TAU
    assert lib.rr_select(None, 8, 1024, 128, f(0.9), FAKE, FAKE, None) == RR_E_NULL
    assert lib.rr_select(FAKE, 0, 1024, 128, f(0.9), FAKE, FAKE, None) == RR_E_SHAPE
    args = [FAKE, FAKE, FAKE, 1024, 8, 2, 128, 128, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, None]
    a = list(args); a[11] = 7
    assert lib.rr_sparse_attn(*a) == RR_E_UNSUPPORTED       # bad output dtype
    a = list(args); a[13] = 1
    assert lib.rr_sparse_attn(*a) == RR_E_WORKSPACE
    a = list(args); a[0] = None
    assert lib.rr_sparse_attn(*a) == RR_E_NULL
    pf = [FAKE, FAKE, FAKE, 1024, 8, 2, 128, 128, 8, f(0.9), FAKE, 1, FAKE, FAKE, FAKE, 1 << 40, None]
    p = list(pf); p[9] = f(-0.1)
    assert lib.rr_prefill(*p) == RR_E_TAU
    p = list(pf); p[8] = 3
    assert lib.rr_prefill(*p) == RR_E_SHAPE
    p = list(pf); p[15] = 10
    assert lib.rr_prefill(*p) == RR_E_WORKSPACE


def test_python_binding_rejects_cpu_tensors():
    import torch
    from long_context_prefill_rr_amd import rr
    q = torch.zeros((128, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        rr.rr_estimate(q, q, 64, 8)


def test_python_binding_rejects_wrong_shapes():
    # The C ABI takes bare pointers and sizes; the binding refuses tensors
    # whose shapes disagree with those sizes before anything reaches the
    # library (CPU tensors of the right shapes then fail the placement check).
    import torch
    from long_context_prefill_rr_amd import rr
    L, Hq, Hkv, d, B, S = 256, 4, 2, 64, 64, 8
    nb = L // B
    bf = dict(dtype=torch.bfloat16)
    q, k, v = torch.zeros((L, Hq, d), **bf), torch.zeros((L, Hkv, d), **bf), torch.zeros((L, Hkv, d), **bf)
    i32 = dict(dtype=torch.int32)
    counts, idx = torch.zeros((Hq, nb), **i32), torch.zeros((Hq, nb, nb), **i32)
    A = torch.zeros((Hq, nb, nb))
    bad = [
        lambda: rr.rr_estimate(q, torch.zeros((L - 8, Hkv, d), **bf), B, S),          # k shorter than q
        lambda: rr.rr_estimate(q, k, B, S, block_scores=torch.zeros((Hq, nb, nb - 1))),
        lambda: rr.rr_estimate(q, k, 0, S),                                             # B = 0
        lambda: rr.rr_xattn_estimate(q, torch.zeros((L, Hkv, d + 8), **bf), B, S),
        lambda: rr.rr_rescue_estimate(q, k, B, block_scores=torch.zeros((Hq + 1, nb, nb))),
        lambda: rr.rr_estimate_materialized(q, k, B, S, block_scores=torch.zeros((Hq, nb, 1))),
        lambda: rr.rr_select(A, L + B, B, 0.9),                                         # nb disagrees with L / B
        lambda: rr.rr_select(A, L, B, 0.9, counts=torch.zeros((Hq, nb + 1), **i32)),
        lambda: rr.rr_select(A, L, B, 0.9, block_idx=torch.zeros((Hq, nb, nb - 1), **i32)),
        lambda: rr.rr_sparse_attn(q, k, torch.zeros((L, Hkv + 1, d), **bf), B, counts, idx),
        lambda: rr.rr_sparse_attn(q, k, v, B, counts[:, :-1], idx),
        lambda: rr.rr_sparse_attn(q, k, v, B, counts, idx, out=torch.zeros((L, Hq, d - 1))),
        lambda: rr.rr_prefill(q, k, v, B, S, 0.9, out=torch.zeros((L - 1, Hq, d), **bf)),
        lambda: rr.rr_prefill(q, k, v, B, S, 0.9, block_idx=idx[:, :, :-1]),
        lambda: rr.rr_mask_quality(counts, idx, counts, idx, A[:, :, :-1], L, B),
        lambda: rr.rr_mask_quality(counts, idx, counts, idx, A, L, B, totals=torch.zeros(4, dtype=torch.float64)),
        lambda: rr.rr_merge_masks(counts, idx, counts, idx[:-1], L, B),
    ]
    for n, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
    good = [
        lambda: rr.rr_estimate(q, k, B, S, block_scores=A),
        lambda: rr.rr_select(A, L, B, 0.9, counts=counts, block_idx=idx),
        lambda: rr.rr_sparse_attn(q, k, v, B, counts, idx),
        lambda: rr.rr_merge_masks(counts, idx, counts, idx, L, B),
    ]
    for call in good:
        with pytest.raises(TypeError):   # right shapes, but host tensors
            call()


def test_mask_quality_validation(lib):
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, 1024, 128, FAKE, FAKE, None]
    a = list(args); a[4] = None
    assert lib.rr_mask_quality(*a) == RR_E_NULL
    a = list(args); a[9] = None
    assert lib.rr_mask_quality(*a) == RR_E_NULL
    a = list(args); a[5] = 0
    assert lib.rr_mask_quality(*a) == RR_E_SHAPE
    a = list(args); a[7] = -1
    assert lib.rr_mask_quality(*a) == RR_E_SHAPE
    a = list(args); a[6] = 128 * 4097
    assert lib.rr_mask_quality(*a) == RR_E_UNSUPPORTED


def test_xattn_estimate_validation(lib):
    def x(L=1024, S=8, B=128, Q=FAKE, ws_bytes=1 << 40, d=128):
        return lib.rr_xattn_estimate(Q, FAKE, L, 8, 2, d, B, S, 0, FAKE, FAKE, ws_bytes, None)
    assert x(Q=None) == RR_E_NULL
    assert x(S=1) == RR_E_UNSUPPORTED       # B/S = 128: no instantiation
    assert x(S=2) == RR_E_UNSUPPORTED       # B/S = 64
    assert x(L=1004) == RR_E_SHAPE          # L % S
    assert x(d=96) == RR_E_UNSUPPORTED
    assert x(ws_bytes=16) == RR_E_WORKSPACE


def test_rescue_and_merge_validation(lib):
    lib.rr_rescue_workspace_bytes.restype = ctypes.c_size_t
    assert lib.rr_rescue_workspace_bytes(1024, 8, 2, 128, 128) == (8 + 2) * 8 * 128 * 4 + 2 * 8 * 4 or \
        lib.rr_rescue_workspace_bytes(1024, 8, 2, 128, 128) >= (8 + 2) * 8 * 128 * 4 + 2 * 8 * 4
    assert lib.rr_rescue_workspace_bytes(1024, 6, 4, 128, 128) == 0          # Hq % Hkv
    r = lambda **kw: lib.rr_rescue_estimate(kw.get("Q", FAKE), FAKE, kw.get("L", 1024), 8, 2,
                                            kw.get("d", 128), kw.get("B", 128), FAKE, FAKE,
                                            kw.get("ws", 1 << 40), None)
    assert r(Q=None) == RR_E_NULL
    assert r(d=96) == RR_E_UNSUPPORTED
    assert r(B=32) == RR_E_UNSUPPORTED
    assert r(ws=16) == RR_E_WORKSPACE
    assert r(L=0) == RR_E_SHAPE
    m = lambda **kw: lib.rr_merge_masks(FAKE, FAKE, kw.get("cb", FAKE), FAKE, 8, kw.get("L", 1024),
                                        128, FAKE, FAKE, None)
    assert m(cb=None) == RR_E_NULL
    assert m(L=0) == RR_E_SHAPE
    assert m(L=128 * 4097) == RR_E_UNSUPPORTED



def test_materialized_estimate_validation(lib):
    # Packed stride scores: Hq * c * P floats, P = c * nb(nb+1)/2.
    L, Hq, Hkv, d, B, S = 1216, 8, 2, 128, 128, 8
    c, nb = B // S, -(-L // B)
    assert lib.rr_stride_scores_count(L, Hq, Hkv, d, B, S) == Hq * c * c * nb * (nb + 1) // 2
    assert lib.rr_stride_scores_count(L, Hq, Hkv, d, B, 64) == 0         # B/S = 2 < 4
    assert lib.rr_stride_scores_count(1004, Hq, Hkv, d, B, S) == 0       # L % S
    ns = L // S
    assert lib.rr_estimate_materialized_workspace_bytes(L, Hq, Hkv, d, B, S) >= 3 * Hkv * ns * d * 2
    assert lib.rr_estimate_materialized_workspace_bytes(L, 6, 4, d, B, S) == 0

    def e(L=1024, S=8, B=128, Q=FAKE, sc=FAKE, ws_bytes=1 << 40, d=128):
        return lib.rr_estimate_materialized(Q, FAKE, L, 8, 2, d, B, S, sc, FAKE, FAKE, ws_bytes, None)
    assert e(Q=None) == RR_E_NULL
    assert e(sc=None) == RR_E_NULL
    assert e(S=64) == RR_E_UNSUPPORTED      # B/S = 2
    assert e(S=128) == RR_E_UNSUPPORTED     # B/S = 1
    assert e(L=1004) == RR_E_SHAPE          # L % S
    assert e(d=96) == RR_E_UNSUPPORTED
    assert e(ws_bytes=16) == RR_E_WORKSPACE
    assert e(L=128 * 4097) == RR_E_UNSUPPORTED
