"""ctypes binding of the fp64 C oracle (test infrastructure only).

Arrays in and out are numpy; bf16 tensors travel as uint16 bit patterns in
the token-major layouts Q [L][Hq][d], K/V [L][Hkv][d].
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile rr_oracle.c with gcc (double precision, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        override = os.environ.get("RR_ORACLE_LIB")  # planted-mistake copies in tests
        if override:
            path = override
        else:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.rro_pool_keys.argtypes = [P, i, i, i, i, P]
        lib.rro_stride_scores.argtypes = [P, P, i, i, i, i, i, i, i, P]
        lib.rro_stride_score_rows.argtypes = [P, P, i, i, i, i, i, P, i, P]
        lib.rro_block_scores.argtypes = [P, P, i, i, i, i, i, i, P, i, P]
        lib.rro_xattn_stride_scores.argtypes = [P, P, i, i, i, i, i, i, i, i, P]
        lib.rro_xattn_block_scores.argtypes = [P, P, i, i, i, i, i, i, i, P, i, P]
        lib.rro_select.argtypes = [P, P, i, i, ctypes.c_double, P, P, P]
        lib.rro_rescue_scores.argtypes = [P, P, i, i, i, i, i, P]
        lib.rro_attention.argtypes = [P, P, P, i, i, i, i, i, P, P, i, P]
        lib.rro_set_threads.argtypes = [i]
        lib.rro_get_threads.restype = i
        for f in ("rro_pool_keys", "rro_stride_scores", "rro_stride_score_rows", "rro_block_scores", "rro_select",
                  "rro_xattn_stride_scores", "rro_xattn_block_scores", "rro_rescue_scores",
                  "rro_attention"):
            getattr(lib, f).restype = i
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a


def _check(rc, name):
    if rc != 0:
        raise ValueError("%s failed with oracle error %d" % (name, rc))


def set_threads(n: int):
    _load().rro_set_threads(int(n))


def get_threads() -> int:
    return _load().rro_get_threads()


def pool_keys(k, S):
    """E1: pooled keys Kbar [Hkv][L/S][d] (float64)."""
    k = _u16(k)
    L, Hkv, d = k.shape
    out = np.empty((Hkv, L // S, d), dtype=np.float64)
    _check(_load().rro_pool_keys(_ptr(k), L, Hkv, d, S, _ptr(out)), "pool_keys")
    return out


def stride_scores(q, k, S, h, i):
    """E2: raw sampled scores s[0..i] of stride row i of query head h."""
    q, k = _u16(q), _u16(k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.empty(i + 1, dtype=np.float64)
    _check(_load().rro_stride_scores(_ptr(q), _ptr(k), L, Hq, Hkv, d, S, h, i, _ptr(out)),
           "stride_scores")
    return out


def stride_score_rows(q, k, S, rows):
    """E2 for many stride rows: rows is a list of (h, i); returns the list of
    score arrays s[0..i] (same values as stride_scores, pooled keys formed once)."""
    q, k = _u16(q), _u16(k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
    lens = rows[:, 1].astype(np.int64) + 1
    out = np.empty(int(lens.sum()), dtype=np.float64)
    _check(_load().rro_stride_score_rows(_ptr(q), _ptr(k), L, Hq, Hkv, d, S, _ptr(rows),
                                         rows.shape[0], _ptr(out)), "stride_score_rows")
    return np.split(out, np.cumsum(lens)[:-1])


def block_scores(q, k, B, S, rows=None):
    """E1-E4: block scores.

    rows=None gives the full [Hq][nb][nb] array; otherwise rows is a list of
    (h, I) pairs and the result is [len(rows)][nb].
    """
    q, k = _u16(q), _u16(k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    nb = -(-L // B)
    full = rows is None
    if full:
        rows = [(h, I) for h in range(Hq) for I in range(nb)]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
    out = np.empty((rows.shape[0], nb), dtype=np.float64)
    _check(_load().rro_block_scores(_ptr(q), _ptr(k), L, Hq, Hkv, d, B, S, _ptr(rows),
                                    rows.shape[0], _ptr(out)), "block_scores")
    return out.reshape(Hq, nb, nb) if full else out


def xattn_stride_scores(q, k, S, h, i, average=False):
    """X1: XAttention antidiagonal scores x[0..i] of stride row i, head h
    (average=True divides each antidiagonal sum by S)."""
    q, k = _u16(q), _u16(k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.empty(i + 1, dtype=np.float64)
    _check(_load().rro_xattn_stride_scores(_ptr(q), _ptr(k), L, Hq, Hkv, d, S, int(average), h,
                                           i, _ptr(out)), "xattn_stride_scores")
    return out


def xattn_block_scores(q, k, B, S, rows=None, average=False):
    """X1 + E3 + E4: XAttention block scores, same layout as block_scores."""
    q, k = _u16(q), _u16(k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    nb = -(-L // B)
    full = rows is None
    if full:
        rows = [(h, I) for h in range(Hq) for I in range(nb)]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
    out = np.empty((rows.shape[0], nb), dtype=np.float64)
    _check(_load().rro_xattn_block_scores(_ptr(q), _ptr(k), L, Hq, Hkv, d, B, S, int(average),
                                          _ptr(rows), rows.shape[0], _ptr(out)),
           "xattn_block_scores")
    return out.reshape(Hq, nb, nb) if full else out


def rescue_scores(q, k, B):
    """R1: RBS rescue-branch scores [Hq][nb][nb] (softmax over J <= I of the
    radius upper-bound logits)."""
    q, k = _u16(q), _u16(k)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    nb = -(-L // B)
    out = np.empty((Hq, nb, nb), dtype=np.float64)
    _check(_load().rro_rescue_scores(_ptr(q), _ptr(k), L, Hq, Hkv, d, B, _ptr(out)),
           "rescue_scores")
    return out


def union_masks(a, b):
    """Combined mask of two selection branches: a block is kept when either
    branch keeps it (RBS-Attention page: the two branches' masks are
    combined)."""
    return (np.asarray(a).astype(bool) | np.asarray(b).astype(bool)).astype(np.uint8)


def select(A, tau, I_of_row=None):
    """E5: Top-tau on block-score rows.

    A is [Hq][nb][nb] (I_of_row omitted) or [n][nb] with I_of_row[n].
    Returns (keep uint8 same shape, counts int32, cbefore float64 same shape).
    """
    A = np.ascontiguousarray(A, dtype=np.float64)
    shape = A.shape
    nb = shape[-1]
    A2 = A.reshape(-1, nb)
    if I_of_row is None:
        I_of_row = np.tile(np.arange(nb, dtype=np.int32), A2.shape[0] // nb)
    I_of_row = np.ascontiguousarray(np.asarray(I_of_row, dtype=np.int32))
    keep = np.empty(A2.shape, dtype=np.uint8)
    cnt = np.empty(A2.shape[0], dtype=np.int32)
    cb = np.empty(A2.shape, dtype=np.float64)
    tau32 = float(np.float32(tau))  # the GPU path receives tau as float32
    _check(_load().rro_select(_ptr(A2), _ptr(I_of_row), A2.shape[0], nb, tau32, _ptr(keep),
                              _ptr(cnt), _ptr(cb)), "select")
    return keep.reshape(shape), cnt.reshape(shape[:-1]), cb.reshape(shape)


def attention(q, k, v, B, mask, toks=None):
    """E6: masked causal attention with GQA.

    mask is uint8 [Hq][nb][nb]; toks=None computes every (t, h) and returns
    [L][Hq][d]; otherwise toks is a list of (h, t) and the result is [n][d].
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    full = toks is None
    if full:
        toks = [(h, t) for t in range(L) for h in range(Hq)]
    toks = np.ascontiguousarray(np.asarray(toks, dtype=np.int32).reshape(-1, 2))
    out = np.empty((toks.shape[0], d), dtype=np.float64)
    _check(_load().rro_attention(_ptr(q), _ptr(k), _ptr(v), L, Hq, Hkv, d, B, _ptr(mask),
                                 _ptr(toks), toks.shape[0], _ptr(out)), "attention")
    return out.reshape(L, Hq, d) if full else out


def mask_from_list(counts, idx, nb):
    """Dense [Hq][nb][nb] mask from a compacted (counts, block index) list."""
    counts = np.asarray(counts)
    idx = np.asarray(idx)
    Hq = counts.shape[0]
    m = np.zeros((Hq, nb, nb), dtype=np.uint8)
    for h in range(Hq):
        for I in range(nb):
            m[h, I, idx[h, I, :counts[h, I]]] = 1
    return m


def list_from_mask(mask):
    """Compacted (counts [Hq][nb], idx [Hq][nb][nb], ascending) from a dense mask."""
    mask = np.asarray(mask)
    Hq, nb, _ = mask.shape
    counts = mask.sum(axis=2).astype(np.int32)
    idx = np.zeros((Hq, nb, nb), dtype=np.int32)
    for h in range(Hq):
        for I in range(nb):
            js = np.nonzero(mask[h, I])[0]
            idx[h, I, :len(js)] = js
    return counts, idx


def mask_quality(mask, ref_mask, mass):
    """Selection quality of a block mask against a reference mask (the
    precision and F1 of selected blocks reported on the RRAttention summary
    page, Key points), written out from the definitions in fp64.

    mask, ref_mask: [Hq][nb][nb] 0/1, only causal entries J <= I count.
    mass: [Hq][nb][nb] block mass (e.g. block_scores with S = 1, the exact
    causal attention mass of each block).

    Returns (rows [Hq][nb][4] = kept, ref, both, share of the row's causal
    mass in the kept blocks; totals [5] = column sums and the minimum share).
    """
    mask = np.asarray(mask).astype(bool)
    ref_mask = np.asarray(ref_mask).astype(bool)
    mass = np.asarray(mass, dtype=np.float64)
    Hq, nb, _ = mask.shape
    rows = np.zeros((Hq, nb, 4), dtype=np.float64)
    for h in range(Hq):
        for I in range(nb):
            t = mask[h, I, :I + 1]
            r = ref_mask[h, I, :I + 1]
            a = mass[h, I, :I + 1]
            w = a.sum()
            rows[h, I, 0] = t.sum()
            rows[h, I, 1] = r.sum()
            rows[h, I, 2] = (t & r).sum()
            rows[h, I, 3] = a[t].sum() / w if w > 0 else 0.0
    flat = rows.reshape(-1, 4)
    totals = np.array([flat[:, 0].sum(), flat[:, 1].sum(), flat[:, 2].sum(), flat[:, 3].sum(),
                       flat[:, 3].min()])
    return rows, totals


def quality_metrics(totals, n_rows):
    """Precision = both/kept, recall = both/ref, F1 = 2 both/(kept + ref),
    and the mean kept mass share per row."""
    kept, ref, both, share, share_min = [float(x) for x in totals]
    return {"precision": both / kept, "recall": both / ref, "f1": 2.0 * both / (kept + ref),
            "mass_recovered_mean": share / n_rows, "mass_recovered_min": share_min}
