"""Small shared helpers for the tests (no method arithmetic here)."""
import numpy as np

from rr_workloads import get_config, generate, bf16_bits_to_f32, f32_to_bf16_bits


def small_workload(kind="llama", L=512, Hq=4, Hkv=2, d=32, B=64, S=8, seed=7, **kw):
    base = {"tiny": 0, "llama": 1, "video": 4}[kind]
    w = get_config(base).with_params(L=L, Hq=Hq, Hkv=Hkv, d=d, B=B, S=S, seed=seed, **kw)
    if kind == "llama":
        w = w.with_params(n_vertical=min(w.n_vertical, max(0, L - w.n_sinks)))
    if kind == "video":
        w = w.with_params(frame_len=kw.get("frame_len", 64))
    return w, generate(w)


def to_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def bf16(x):
    """float array -> bf16 bit patterns (round to nearest even)."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
