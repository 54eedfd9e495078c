"""ctypes binding of librr.so: the same calls as the C ABI (include/rr.h).

Every function only checks tensor shapes, placement, dtype and contiguity,
allocates outputs and workspace with torch when the caller does not pass them,
and forwards device pointers plus the current HIP stream.  All arithmetic runs
in the library's kernels.  The shape checks matter: the C ABI takes bare
pointers and sizes, so a tensor smaller than the sizes say would be read or
written out of bounds on the device.

Layouts: q [L][Hq][d], k and v [L][Hkv][d], all torch.bfloat16 on the GPU.
"""
import ctypes
import os

import torch

RR_OUT_BF16 = 0
RR_OUT_F32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librr.so")
_lib = None

_STATUS = {0: "RR_OK", 1: "RR_E_NULL", 2: "RR_E_SHAPE", 3: "RR_E_TAU", 4: "RR_E_WORKSPACE",
           5: "RR_E_UNSUPPORTED", 6: "RR_E_HIP"}


class RRError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        msg = _load().rr_status_str(code).decode() if _lib is not None else _STATUS.get(code, "?")
        super().__init__("%s: %s (status %d)" % (where, msg, code))


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load librr.so (raises if it has not been built)."""
    return _load()


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("librr.so not found at %s: build it with "
                              "`python -m long_context_prefill_rr_amd.build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, i, z, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        lib.rr_status_str.argtypes = [i]
        lib.rr_status_str.restype = ctypes.c_char_p
        lib.rr_abi_version.restype = i
        lib.rr_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.rr_workspace_bytes.restype = z
        lib.rr_estimate_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.rr_estimate_workspace_bytes.restype = z
        lib.rr_sparse_attn_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.rr_sparse_attn_workspace_bytes.restype = z
        lib.rr_prefill_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.rr_prefill_workspace_bytes.restype = z
        lib.rr_estimate.argtypes = [P, P, i, i, i, i, i, i, P, P, z, P]
        lib.rr_select.argtypes = [P, i, i, i, f, P, P, P]
        lib.rr_sparse_attn.argtypes = [P, P, P, i, i, i, i, i, P, P, P, i, P, z, P]
        lib.rr_prefill.argtypes = [P, P, P, i, i, i, i, i, i, f, P, i, P, P, P, z, P]
        lib.rr_noalloc_scratch_bytes.argtypes = []
        lib.rr_noalloc_scratch_bytes.restype = z
        lib.rr_prefill_noalloc.argtypes = [P, P, P, i, i, i, i, i, i, f, P, i, P, P, P]
        lib.rr_mask_quality.argtypes = [P, P, P, P, P, i, i, i, P, P, P]
        lib.rr_xattn_estimate.argtypes = [P, P, i, i, i, i, i, i, i, P, P, z, P]
        lib.rr_rescue_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.rr_rescue_workspace_bytes.restype = z
        lib.rr_rescue_estimate.argtypes = [P, P, i, i, i, i, i, P, P, z, P]
        lib.rr_merge_masks.argtypes = [P, P, P, P, i, i, i, P, P, P]
        lib.rr_stride_scores_count.argtypes = [i, i, i, i, i, i]
        lib.rr_stride_scores_count.restype = ctypes.c_longlong
        lib.rr_estimate_materialized_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.rr_estimate_materialized_workspace_bytes.restype = z
        lib.rr_estimate_materialized.argtypes = [P, P, i, i, i, i, i, i, P, P, P, z, P]
        for name in ("rr_estimate", "rr_select", "rr_sparse_attn", "rr_prefill", "rr_prefill_noalloc",
                     "rr_mask_quality",
                     "rr_xattn_estimate", "rr_rescue_estimate", "rr_merge_masks",
                     "rr_estimate_materialized"):
            getattr(lib, name).restype = i
        _lib = lib
    return _lib


def _stream_ptr(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, name, shape):
    """Refuse a tensor whose shape differs from the one the call reads or writes."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _nblocks(L, B):
    if B <= 0 or L <= 0:
        raise ValueError("L and B must be positive (L=%d, B=%d)" % (L, B))
    return -(-L // B)


def _qkv(q, k, v=None):
    """(L, Hq, Hkv, d) from q [L][Hq][d]; k (and v) must be [L][Hkv][d]."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be 3-D ([L][heads][d])")
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    _shape(k, "k", (L, Hkv, d))
    if v is not None:
        _shape(v, "v", (L, Hkv, d))
    return L, Hq, Hkv, d


def _check(rc, where):
    if rc != 0:
        raise RRError(rc, where)


def workspace_bytes(L, Hq, Hkv, d, B, S):
    """Bytes of one workspace that serves every call on this shape (0: invalid)."""
    return _load().rr_workspace_bytes(L, Hq, Hkv, d, B, S)


def estimate_workspace_bytes(L, Hq, Hkv, d, B, S):
    return _load().rr_estimate_workspace_bytes(L, Hq, Hkv, d, B, S)


def sparse_attn_workspace_bytes(L, Hq, Hkv, d, B):
    return _load().rr_sparse_attn_workspace_bytes(L, Hq, Hkv, d, B)


def rescue_workspace_bytes(L, Hq, Hkv, d, B):
    return _load().rr_rescue_workspace_bytes(L, Hq, Hkv, d, B)


def prefill_workspace_bytes(L, Hq, Hkv, d, B, S):
    return _load().rr_prefill_workspace_bytes(L, Hq, Hkv, d, B, S)


def _workspace(nbytes, device, ws):
    if ws is None:
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small: %d < %d bytes" % (ws.numel() * ws.element_size(), nbytes))
    return ws


def rr_estimate(q, k, B, S, block_scores=None, ws=None, stream=None):
    """Block scores [Hq][nb][nb] (fp32) of the round-robin estimate."""
    L, Hq, Hkv, d = _qkv(q, k)
    nb = _nblocks(L, B)
    _shape(block_scores, "block_scores", (Hq, nb, nb))
    if block_scores is None:
        block_scores = torch.empty((Hq, nb, nb), dtype=torch.float32, device=q.device)
    lib = _load()
    ws = _workspace(lib.rr_estimate_workspace_bytes(L, Hq, Hkv, d, B, S), q.device, ws)
    rc = lib.rr_estimate(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), L, Hq, Hkv,
                         d, B, S, _dev(block_scores, "block_scores", torch.float32),
                         _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(rc, "rr_estimate")
    return block_scores


def stride_scores_count(L, Hq, Hkv, d, B, S):
    """Floats of rr_estimate_materialized's stride-score buffer (0: unsupported shape)."""
    return _load().rr_stride_scores_count(L, Hq, Hkv, d, B, S)


def rr_estimate_materialized(q, k, B, S, stride_scores=None, block_scores=None, ws=None,
                             stream=None):
    """(stride_scores, block_scores): every stride score written to memory
    (packed layout of include/rr.h, base-2 logits, -inf above the diagonal),
    then pooled; block_scores as for rr_estimate."""
    L, Hq, Hkv, d = _qkv(q, k)
    nb = _nblocks(L, B)
    _shape(block_scores, "block_scores", (Hq, nb, nb))
    lib = _load()
    n = lib.rr_stride_scores_count(L, Hq, Hkv, d, B, S)
    if stride_scores is None:
        stride_scores = torch.empty(max(n, 1), dtype=torch.float32, device=q.device)
    if block_scores is None:
        block_scores = torch.empty((Hq, nb, nb), dtype=torch.float32, device=q.device)
    ws = _workspace(lib.rr_estimate_materialized_workspace_bytes(L, Hq, Hkv, d, B, S), q.device, ws)
    if stride_scores.numel() < n:
        raise ValueError("stride_scores holds %d floats, %d needed" % (stride_scores.numel(), n))
    rc = lib.rr_estimate_materialized(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), L,
                                      Hq, Hkv, d, B, S,
                                      _dev(stride_scores, "stride_scores", torch.float32),
                                      _dev(block_scores, "block_scores", torch.float32),
                                      _dev(ws, "ws"), ws.numel() * ws.element_size(),
                                      _stream_ptr(stream))
    _check(rc, "rr_estimate_materialized")
    return stride_scores, block_scores


def rr_xattn_estimate(q, k, B, S, block_scores=None, ws=None, stream=None, average=False):
    """Block scores [Hq][nb][nb] (fp32) of XAttention's antidiagonal estimate
    (average=True: antidiagonal mean instead of sum)."""
    L, Hq, Hkv, d = _qkv(q, k)
    nb = _nblocks(L, B)
    _shape(block_scores, "block_scores", (Hq, nb, nb))
    if block_scores is None:
        block_scores = torch.empty((Hq, nb, nb), dtype=torch.float32, device=q.device)
    lib = _load()
    ws = _workspace(lib.rr_estimate_workspace_bytes(L, Hq, Hkv, d, B, S), q.device, ws)
    rc = lib.rr_xattn_estimate(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), L, Hq,
                               Hkv, d, B, S, int(bool(average)),
                               _dev(block_scores, "block_scores", torch.float32),
                               _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(rc, "rr_xattn_estimate")
    return block_scores


def rr_select(block_scores, L, B, tau, counts=None, block_idx=None, stream=None):
    """Top-tau selection: (counts [Hq][nb], block_idx [Hq][nb][nb]) int32."""
    if block_scores.dim() != 3:
        raise ValueError("block_scores must be 3-D ([Hq][nb][nb])")
    Hq = block_scores.shape[0]
    nb = _nblocks(L, B)
    _shape(block_scores, "block_scores", (Hq, nb, nb))
    _shape(counts, "counts", (Hq, nb))
    _shape(block_idx, "block_idx", (Hq, nb, nb))
    dev = block_scores.device
    if counts is None:
        counts = torch.empty((Hq, nb), dtype=torch.int32, device=dev)
    if block_idx is None:
        block_idx = torch.empty((Hq, nb, nb), dtype=torch.int32, device=dev)
    rc = _load().rr_select(_dev(block_scores, "block_scores", torch.float32), Hq, L, B,
                           float(tau), _dev(counts, "counts", torch.int32),
                           _dev(block_idx, "block_idx", torch.int32), _stream_ptr(stream))
    _check(rc, "rr_select")
    return counts, block_idx


def _out_code(out_dtype):
    if out_dtype == torch.float32:
        return RR_OUT_F32
    if out_dtype == torch.bfloat16:
        return RR_OUT_BF16
    raise TypeError("output dtype must be float32 or bfloat16")


def rr_sparse_attn(q, k, v, B, counts, block_idx, out=None, out_dtype=torch.float32, ws=None,
                   stream=None):
    """Causal block-sparse GQA attention over the listed blocks -> O [L][Hq][d]."""
    L, Hq, Hkv, d = _qkv(q, k, v)
    nb = _nblocks(L, B)
    _shape(counts, "counts", (Hq, nb))
    _shape(block_idx, "block_idx", (Hq, nb, nb))
    _shape(out, "out", (L, Hq, d))
    if out is None:
        out = torch.empty((L, Hq, d), dtype=out_dtype, device=q.device)
    code = _out_code(out.dtype)
    lib = _load()
    ws = _workspace(lib.rr_sparse_attn_workspace_bytes(L, Hq, Hkv, d, B), q.device, ws)
    rc = lib.rr_sparse_attn(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                            _dev(v, "v", torch.bfloat16), L, Hq, Hkv, d, B,
                            _dev(counts, "counts", torch.int32),
                            _dev(block_idx, "block_idx", torch.int32), _dev(out, "out"), code,
                            _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(rc, "rr_sparse_attn")
    return out


def rr_prefill(q, k, v, B, S, tau, out=None, out_dtype=torch.bfloat16, counts=None,
               block_idx=None, ws=None, stream=None):
    """The whole sparse prefill: returns (O, counts, block_idx)."""
    L, Hq, Hkv, d = _qkv(q, k, v)
    nb = _nblocks(L, B)
    _shape(out, "out", (L, Hq, d))
    _shape(counts, "counts", (Hq, nb))
    _shape(block_idx, "block_idx", (Hq, nb, nb))
    dev = q.device
    if out is None:
        out = torch.empty((L, Hq, d), dtype=out_dtype, device=dev)
    if counts is None:
        counts = torch.empty((Hq, nb), dtype=torch.int32, device=dev)
    if block_idx is None:
        block_idx = torch.empty((Hq, nb, nb), dtype=torch.int32, device=dev)
    code = _out_code(out.dtype)
    lib = _load()
    ws = _workspace(lib.rr_prefill_workspace_bytes(L, Hq, Hkv, d, B, S), dev, ws)
    rc = lib.rr_prefill(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                        _dev(v, "v", torch.bfloat16), L, Hq, Hkv, d, B, S, float(tau),
                        _dev(out, "out"), code, _dev(counts, "counts", torch.int32),
                        _dev(block_idx, "block_idx", torch.int32), _dev(ws, "ws"),
                        ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(rc, "rr_prefill")
    return out, counts, block_idx


def noalloc_scratch_bytes():
    """Bytes of the library-owned workspace rr_prefill_noalloc uses on each GPU."""
    return _load().rr_noalloc_scratch_bytes()


def rr_prefill_noalloc(q, k, v, B, S, tau, out=None, out_dtype=torch.bfloat16, counts=None,
                       block_idx=None, stream=None):
    """rr_prefill with the library's own workspace (no workspace argument, no
    device allocation inside the call): returns (O, counts, block_idx).  Pass
    out, counts and block_idx to keep this wrapper from allocating them."""
    L, Hq, Hkv, d = _qkv(q, k, v)
    nb = _nblocks(L, B)
    _shape(out, "out", (L, Hq, d))
    _shape(counts, "counts", (Hq, nb))
    _shape(block_idx, "block_idx", (Hq, nb, nb))
    dev = q.device
    if out is None:
        out = torch.empty((L, Hq, d), dtype=out_dtype, device=dev)
    if counts is None:
        counts = torch.empty((Hq, nb), dtype=torch.int32, device=dev)
    if block_idx is None:
        block_idx = torch.empty((Hq, nb, nb), dtype=torch.int32, device=dev)
    code = _out_code(out.dtype)
    rc = _load().rr_prefill_noalloc(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16),
                                    _dev(v, "v", torch.bfloat16), L, Hq, Hkv, d, B, S, float(tau),
                                    _dev(out, "out"), code, _dev(counts, "counts", torch.int32),
                                    _dev(block_idx, "block_idx", torch.int32), _stream_ptr(stream))
    _check(rc, "rr_prefill_noalloc")
    return out, counts, block_idx


def rr_mask_quality(counts, block_idx, ref_counts, ref_block_idx, mass, L, B, rows=None,
                    totals=None, stream=None):
    """Per-row (kept, ref, both, kept mass share) [Hq][nb][4] fp32 and their
    totals [5] fp64 (sums of the four columns, then the minimum share)."""
    if counts.dim() != 2:
        raise ValueError("counts must be 2-D ([Hq][nb])")
    Hq = counts.shape[0]
    nb = _nblocks(L, B)
    _shape(counts, "counts", (Hq, nb))
    _shape(block_idx, "block_idx", (Hq, nb, nb))
    _shape(ref_counts, "ref_counts", (Hq, nb))
    _shape(ref_block_idx, "ref_block_idx", (Hq, nb, nb))
    _shape(mass, "mass", (Hq, nb, nb))
    _shape(rows, "rows", (Hq, nb, 4))
    _shape(totals, "totals", (5,))
    dev = counts.device
    if rows is None:
        rows = torch.empty((Hq, nb, 4), dtype=torch.float32, device=dev)
    if totals is None:
        totals = torch.empty(5, dtype=torch.float64, device=dev)
    rc = _load().rr_mask_quality(_dev(counts, "counts", torch.int32),
                                 _dev(block_idx, "block_idx", torch.int32),
                                 _dev(ref_counts, "ref_counts", torch.int32),
                                 _dev(ref_block_idx, "ref_block_idx", torch.int32),
                                 _dev(mass, "mass", torch.float32), Hq, L, B,
                                 _dev(rows, "rows", torch.float32),
                                 _dev(totals, "totals", torch.float64), _stream_ptr(stream))
    _check(rc, "rr_mask_quality")
    return rows, totals


def quality_summary(totals, n_rows):
    """Precision, recall, F1 and mean / minimum kept mass share from the
    totals of rr_mask_quality (host arithmetic on five numbers)."""
    kept, ref, both, share, share_min = [float(x) for x in totals]
    return {"precision": both / kept if kept else 0.0,
            "recall": both / ref if ref else 0.0,
            "f1": 2.0 * both / (kept + ref) if kept + ref else 0.0,
            "mass_recovered_mean": share / n_rows if n_rows else 0.0,
            "mass_recovered_min": share_min,
            "kept_blocks": int(round(kept)), "reference_blocks": int(round(ref)),
            "common_blocks": int(round(both))}


def rr_rescue_estimate(q, k, B, block_scores=None, ws=None, stream=None):
    """Rescue-branch block scores [Hq][nb][nb] (fp32, rows sum to 1)."""
    L, Hq, Hkv, d = _qkv(q, k)
    nb = _nblocks(L, B)
    _shape(block_scores, "block_scores", (Hq, nb, nb))
    if block_scores is None:
        block_scores = torch.empty((Hq, nb, nb), dtype=torch.float32, device=q.device)
    lib = _load()
    ws = _workspace(lib.rr_rescue_workspace_bytes(L, Hq, Hkv, d, B), q.device, ws)
    rc = lib.rr_rescue_estimate(_dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16), L, Hq,
                                Hkv, d, B, _dev(block_scores, "block_scores", torch.float32),
                                _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(rc, "rr_rescue_estimate")
    return block_scores


def rr_merge_masks(counts_a, block_idx_a, counts_b, block_idx_b, L, B, counts=None,
                   block_idx=None, stream=None):
    """Union of two block lists: (counts [Hq][nb], block_idx [Hq][nb][nb])."""
    if counts_a.dim() != 2:
        raise ValueError("counts_a must be 2-D ([Hq][nb])")
    Hq = counts_a.shape[0]
    nb = _nblocks(L, B)
    for t, name in ((counts_a, "counts_a"), (counts_b, "counts_b"), (counts, "counts")):
        _shape(t, name, (Hq, nb))
    for t, name in ((block_idx_a, "block_idx_a"), (block_idx_b, "block_idx_b"), (block_idx, "block_idx")):
        _shape(t, name, (Hq, nb, nb))
    dev = counts_a.device
    if counts is None:
        counts = torch.empty((Hq, nb), dtype=torch.int32, device=dev)
    if block_idx is None:
        block_idx = torch.empty((Hq, nb, nb), dtype=torch.int32, device=dev)
    rc = _load().rr_merge_masks(_dev(counts_a, "counts_a", torch.int32),
                                _dev(block_idx_a, "block_idx_a", torch.int32),
                                _dev(counts_b, "counts_b", torch.int32),
                                _dev(block_idx_b, "block_idx_b", torch.int32), Hq, L, B,
                                _dev(counts, "counts", torch.int32),
                                _dev(block_idx, "block_idx", torch.int32), _stream_ptr(stream))
    _check(rc, "rr_merge_masks")
    return counts, block_idx

