"""Deterministic synthetic Q/K/V generator (bf16 bit patterns).

Recipe (per workload, seed s):

* Five independent numpy streams are spawned from ``SeedSequence([s, 0x5252])``:
  0 means, 1 Q noise, 2 K noise, 3 V, 4 special positions.
* Token-major layouts: Q ``[L][Hq][d]``, K and V ``[L][Hkv][d]``; query head h
  reads kv-head ``h // (Hq // Hkv)``.
* kind "tiny":  one mean vector mu_g ~ N(0,1)^d per kv-head;
  Q[t,h] = mu_g(h) + 0.5 N(0,1),  K[t,g] = mu_g + 0.5 N(0,1).
* kind "llama": as "tiny"; after RoPE, keys of the first ``n_sinks`` tokens
  (every kv-head) and of ``n_vertical`` distinct positions per kv-head drawn
  uniformly from [n_sinks, L) are multiplied by ``key_scale`` (x4).
* kind "video": tokens form frames of ``frame_len``; per kv-head a frame
  vector F_f ~ N(0,1)^d and a slot vector P_s ~ N(0,1)^d, shared across
  frames; K = F_f + P_s + 0.5 N, Q = F_f + P_s + 0.5 N with independent noise.
* RoPE (rotate-half, theta_f = base^(-2f/d), position t) is applied to Q and K
  before any key scaling (a scale commutes with the rotation).
* V ~ N(0,1).
* Noise is drawn in float32 in chunks of 4096 tokens; arithmetic is float32
  with cos/sin computed in float64; the result is rounded to bf16 with
  round-to-nearest-even.

Nothing here scores, normalises, selects or attends: it only makes inputs.
"""
import numpy as np

from .configs import Workload

CHUNK = 4096


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rope(x: np.ndarray, t0: int, base: float) -> np.ndarray:
    """Rotate-half RoPE on x[tokens][heads][d] whose first token is t0."""
    n, _, d = x.shape
    half = d // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.arange(t0, t0 + n, dtype=np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang).astype(np.float32)[:, None, :]
    sin = np.sin(ang).astype(np.float32)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = x1 * cos - x2 * sin
    out[..., half:] = x2 * cos + x1 * sin
    return out


def generate(w: Workload, seed: int = None):
    """Return dict(q, k, v, sinks, verticals) for workload ``w``.

    q: uint16 [L][Hq][d], k/v: uint16 [L][Hkv][d] (bf16 bit patterns),
    sinks: int array of scaled leading positions,
    verticals: int array [Hkv][n_vertical] of scaled positions.
    """
    seed = w.seed if seed is None else seed
    L, Hq, Hkv, d, G = w.L, w.Hq, w.Hkv, w.d, w.G
    assert Hq % Hkv == 0
    streams = [np.random.default_rng(s)
               for s in np.random.SeedSequence([seed, 0x5252]).spawn(5)]
    r_mean, r_q, r_k, r_v, r_sp = streams
    g_of_h = np.arange(Hq) // G

    if w.kind in ("tiny", "llama"):
        mu = r_mean.standard_normal((Hkv, d)).astype(np.float32)
        frames = slots = None
    elif w.kind == "video":
        nf = -(-L // w.frame_len)
        frames = r_mean.standard_normal((Hkv, nf, d)).astype(np.float32)
        slots = r_mean.standard_normal((Hkv, w.frame_len, d)).astype(np.float32)
        mu = None
    else:
        raise ValueError(w.kind)

    sinks = np.arange(min(w.n_sinks, L))
    if w.n_vertical > 0:
        span = L - w.n_sinks
        verticals = np.stack([
            np.sort(r_sp.choice(span, size=min(w.n_vertical, span), replace=False)) + w.n_sinks
            for _ in range(Hkv)])
    else:
        verticals = np.zeros((Hkv, 0), dtype=np.int64)

    q = np.empty((L, Hq, d), dtype=np.uint16)
    k = np.empty((L, Hkv, d), dtype=np.uint16)
    v = np.empty((L, Hkv, d), dtype=np.uint16)
    std = np.float32(w.noise_std)
    for t0 in range(0, L, CHUNK):
        n = min(CHUNK, L - t0)
        t = np.arange(t0, t0 + n)
        if mu is not None:
            base_k = np.broadcast_to(mu[None, :, :], (n, Hkv, d))
        else:
            base_k = (frames[:, t // w.frame_len, :] + slots[:, t % w.frame_len, :]).transpose(1, 0, 2)
        base_q = base_k[:, g_of_h, :]
        qc = base_q + std * r_q.standard_normal((n, Hq, d), dtype=np.float32)
        kc = base_k + std * r_k.standard_normal((n, Hkv, d), dtype=np.float32)
        vc = r_v.standard_normal((n, Hkv, d), dtype=np.float32)
        qc = _rope(qc.astype(np.float32), t0, w.rope_base)
        kc = _rope(kc.astype(np.float32), t0, w.rope_base)
        if w.kind == "llama":
            scale = np.ones((n, Hkv), dtype=np.float32)
            in_chunk = (sinks >= t0) & (sinks < t0 + n)
            scale[sinks[in_chunk] - t0, :] = w.key_scale
            for g in range(Hkv):
                vv = verticals[g]
                m = (vv >= t0) & (vv < t0 + n)
                scale[vv[m] - t0, g] = w.key_scale
            kc = kc * scale[:, :, None]
        q[t0:t0 + n] = f32_to_bf16_bits(qc)
        k[t0:t0 + n] = f32_to_bf16_bits(kc)
        v[t0:t0 + n] = f32_to_bf16_bits(vc)
    return dict(q=q, k=k, v=v, sinks=sinks, verticals=verticals)
