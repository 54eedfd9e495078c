"""Workload shapes.

The attention shapes follow the models the RRAttention pages evaluate on
(RRAttention summary page, "Key points": LLaMA-3.1-8B-Instruct and Qwen at
8K-128K; XAttention review page, "Experimental setup": Llama-3.1-8B-Instruct
and QwenVL-2-7B).  Block size B=128 and stride S=8 are the method's defaults,
S=16 the other recommended stride (RRAttention summary page, "Key points").

Five workloads, indexed 0..4:

  0  tiny-1k        8/8 heads, d=64,  L=1024,   S=8,  tau=0.9
  1  llama8b-8k     32/8 heads, d=128, L=8192,   S=8,  tau=0.9
  2  llama8b-32k    32/8 heads, d=128, L=32768,  S=8,  tau=0.9 (+ S/tau sweep)
  3  llama8b-128k   32/8 heads, d=128, L=131072, S=8,  tau=0.9 (headline)
  4  qwen2-7b-video 28/4 heads, d=128, L=65536 (256 frames x 256), S=16, tau=0.9
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    Hq: int
    Hkv: int
    d: int
    L: int
    B: int
    S: int
    tau: float
    rope_base: float
    kind: str                 # "tiny" | "llama" | "video"
    seed: int
    n_sinks: int = 0          # leading tokens whose keys are scaled
    n_vertical: int = 0       # random key positions per kv-head that are scaled
    key_scale: float = 4.0    # scale applied to sink / vertical keys
    frame_len: int = 256      # tokens per frame for the video-like layout
    noise_std: float = 0.5
    sweep: Tuple[Tuple[int, float], ...] = field(default_factory=tuple)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def nb(self) -> int:
        return -(-self.L // self.B)

    @property
    def ns(self) -> int:
        return self.L // self.S

    def with_params(self, **kw) -> "Workload":
        return replace(self, **kw)


CONFIGS = (
    Workload(0, "tiny-1k", Hq=8, Hkv=8, d=64, L=1024, B=128, S=8, tau=0.9,
             rope_base=1.0e4, kind="tiny", seed=0),
    Workload(1, "llama8b-8k", Hq=32, Hkv=8, d=128, L=8192, B=128, S=8, tau=0.9,
             rope_base=5.0e5, kind="llama", seed=1, n_sinks=4, n_vertical=16),
    Workload(2, "llama8b-32k", Hq=32, Hkv=8, d=128, L=32768, B=128, S=8, tau=0.9,
             rope_base=5.0e5, kind="llama", seed=2, n_sinks=4, n_vertical=16,
             sweep=tuple((s, t) for s in (8, 16) for t in (0.8, 0.9, 0.95))),
    Workload(3, "llama8b-128k", Hq=32, Hkv=8, d=128, L=131072, B=128, S=8, tau=0.9,
             rope_base=5.0e5, kind="llama", seed=3, n_sinks=4, n_vertical=16),
    Workload(4, "qwen2-7b-video-64k", Hq=28, Hkv=4, d=128, L=65536, B=128, S=16,
             tau=0.9, rope_base=1.0e6, kind="video", seed=4, frame_len=256),
)


def get_config(key) -> Workload:
    """Look a workload up by index (0..4) or by name."""
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS:
        if c.name == key:
            return c
    raise KeyError(key)
