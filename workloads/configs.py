"""Registry of the five workloads the attention block is checked and timed on.

Pure data: shapes, dtypes, per-layer (type, theta, scale) and the query scale.
Layer types are spelled out per workload; nothing here computes any part of
the attention block.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

LOCAL_SLIDING = "LOCAL_SLIDING"
GLOBAL = "GLOBAL"


@dataclass(frozen=True)
class Layer:
    attn_type: str          # LOCAL_SLIDING or GLOBAL
    rope_theta: float
    rope_scale: float


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    mode: str               # "prefill" or "decode"
    dtype: str              # "f32" or "bf16"
    B: int
    T: int
    D: int
    H: int
    H_kv: int
    d_h: int
    window: int
    query_scale: float
    layers: Tuple[Layer, ...]
    # prefill: number of right-padded key positions per batch row (0 = none)
    pad_tail: Tuple[int, ...] = ()
    # decode: cache capacity S and the range the per-row lengths are drawn from
    cache_len: int = 0
    len_range: Tuple[int, int] = (0, 0)
    notes: str = ""

    @property
    def G(self) -> int:
        return self.H // self.H_kv

    def kv_valid_len(self) -> Optional[Tuple[int, ...]]:
        if not self.pad_tail:
            return None
        return tuple(self.T - p for p in self.pad_tail)


_L = lambda: Layer(LOCAL_SLIDING, 1e4, 1.0)  # noqa: E731

WORKLOADS = {
    1: Workload(
        1, "local-fp32-T128", "prefill", "f32",
        B=1, T=128, D=256, H=4, H_kv=1, d_h=64, window=32,
        query_scale=64 ** -0.5, layers=(_L(),),
        notes="single local layer, fp32, causal, no cache"),
    2: Workload(
        2, "gemma3-1b-shaped-LG-T4096", "prefill", "bf16",
        B=1, T=4096, D=1152, H=4, H_kv=1, d_h=256, window=512,
        query_scale=256 ** -0.5,
        layers=(_L(), Layer(GLOBAL, 1e6, 1.0)),
        notes="one local and one global layer, multi-query, causal"),
    3: Workload(
        3, "gemma3-4b-like-LLLLLG-B4-T8192", "prefill", "bf16",
        B=4, T=8192, D=2560, H=8, H_kv=4, d_h=256, window=1024,
        query_scale=256 ** -0.5,
        layers=(_L(), _L(), _L(), _L(), _L(), Layer(GLOBAL, 1e6, 8.0)),
        # last floor(0.05 * 8192) = 409 key positions of rows 1 and 3 padded
        pad_tail=(0, 409, 0, 409),
        notes="six-layer tile, GQA G=2, causal plus key padding"),
    4: Workload(
        4, "gemma3-27b-shaped-LG-T32768", "prefill", "bf16",
        B=1, T=32768, D=5376, H=32, H_kv=16, d_h=128, window=1024,
        query_scale=(5376 / 32) ** -0.5,
        layers=(_L(), Layer(GLOBAL, 1e6, 8.0)),
        notes="one local and one global layer, d_h=128, alpha=168^-1/2"),
    5: Workload(
        5, "gemma3-12b-like-decode-B16", "decode", "bf16",
        B=16, T=1, D=3840, H=16, H_kv=8, d_h=256, window=1024,
        query_scale=256 ** -0.5,
        layers=(Layer(GLOBAL, 1e6, 8.0), _L()),
        cache_len=131072, len_range=(1024, 131072),
        notes="one decode token per row against a left-aligned bf16 cache"),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(changes)
    return Workload(**d)
