"""Seeded input generation for the attention-block workloads.

Every random draw comes from ``numpy.random.default_rng([cfg_id, layer_id, tag])``
in float64 and is then rounded to the workload dtype (round-to-nearest-even via
torch). The only exception is the decode KV cache at full size (about 4.3e9
values per tensor), which is drawn on the device with a seeded torch generator;
both sides then read the same stored bytes.

Distributions (per workload description):
  x ~ N(0, 1); W_q, W_kv, W_o ~ N(0, std D^-1/2); gamma_Q, gamma_K ~ N(0, std 0.1);
  segment_pos = 0..T-1 in prefill; decode positions = cache length - 1.
Cached keys are unit-RMS Gaussian vectors. The workload asks for RMS-normalised
Gaussian keys with RoPE applied; a rotation maps an isotropic Gaussian vector
to another one of the same law and keeps its RMS, so drawing unit-RMS Gaussian
vectors directly samples exactly that distribution without any attention
arithmetic here. Cached values are unit-RMS Gaussian vectors as well.
"""

from __future__ import annotations

import numpy as np
import torch

from .configs import Workload

TAG_X, TAG_WQ, TAG_WKV, TAG_WO, TAG_GQ, TAG_GK, TAG_LEN, TAG_KC, TAG_VC = range(9)

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def rng(cfg_id: int, layer_id: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([cfg_id, layer_id, tag])


def _normal(cfg_id, layer_id, tag, shape, std=1.0) -> np.ndarray:
    return rng(cfg_id, layer_id, tag).standard_normal(size=shape) * std


def to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Round an fp64 array to the workload dtype (CPU tensor)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(TORCH_DTYPE[dtype])


def layer_weights(w: Workload, layer_id: int) -> dict:
    """Weights of one layer, output-major: w_q [H*d_h, D], w_kv [2*H_kv*d_h, D]
    (K heads then V heads), w_o [D, H*d_h]; gamma_q, gamma_k [d_h]."""
    std = w.D ** -0.5
    c = w.cfg_id
    return dict(
        w_q=to_dtype(_normal(c, layer_id, TAG_WQ, (w.H * w.d_h, w.D), std), w.dtype),
        w_kv=to_dtype(_normal(c, layer_id, TAG_WKV, (2 * w.H_kv * w.d_h, w.D), std), w.dtype),
        w_o=to_dtype(_normal(c, layer_id, TAG_WO, (w.D, w.H * w.d_h), std), w.dtype),
        gamma_q=to_dtype(_normal(c, layer_id, TAG_GQ, (w.d_h,), 0.1), w.dtype),
        gamma_k=to_dtype(_normal(c, layer_id, TAG_GK, (w.d_h,), 0.1), w.dtype),
    )


def prefill_x(w: Workload) -> torch.Tensor:
    """x [B,T,D]; every layer of a workload takes the same x."""
    return to_dtype(_normal(w.cfg_id, 0, TAG_X, (w.B, w.T, w.D)), w.dtype)


def prefill_positions(w: Workload) -> torch.Tensor:
    return torch.arange(w.T, dtype=torch.int32).repeat(w.B, 1).contiguous()


def prefill_kv_valid_len(w: Workload):
    lens = w.kv_valid_len()
    return None if lens is None else torch.tensor(lens, dtype=torch.int32)


def prefill_inputs(w: Workload, layer_id: int) -> dict:
    d = layer_weights(w, layer_id)
    d.update(x=prefill_x(w), segment_pos=prefill_positions(w),
             kv_valid_len=prefill_kv_valid_len(w))
    return d


def decode_lengths(w: Workload) -> np.ndarray:
    """Per-row cache length L_b ~ U{lo..hi} (after the step's own write)."""
    lo, hi = w.len_range
    return rng(w.cfg_id, 0, TAG_LEN).integers(lo, hi, size=w.B, endpoint=True)


def decode_inputs(w: Workload, layer_id: int, lengths=None) -> dict:
    """x [B,1,D] and segment_pos [B,1] = L_b - 1, plus this layer's weights."""
    lens = decode_lengths(w) if lengths is None else np.asarray(lengths)
    d = layer_weights(w, layer_id)
    d.update(x=to_dtype(_normal(w.cfg_id, layer_id, TAG_X, (w.B, 1, w.D)), w.dtype),
             segment_pos=torch.tensor(lens - 1, dtype=torch.int32).reshape(w.B, 1),
             lengths=lens)
    return d


def _unit_rms(g: torch.Tensor) -> torch.Tensor:
    return g / torch.sqrt(torch.mean(g * g, dim=-1, keepdim=True))


def decode_cache(w: Workload, layer_id: int, lengths, device="cpu",
                 poison: bool = True):
    """K and V caches [B,S,H_kv,d_h] in the workload dtype.

    Slots 0..L_b-2 hold unit-RMS Gaussian vectors; slots L_b-1.. (the slot the
    decode step writes, and everything after it) hold NaN when ``poison``.
    Drawn per batch row with a seeded torch generator on ``device``.
    """
    S, Hk, d_h = w.cache_len, w.H_kv, w.d_h
    dt = TORCH_DTYPE[w.dtype]
    caches = []
    for tag in (TAG_KC, TAG_VC):
        c = torch.empty((w.B, S, Hk, d_h), dtype=dt, device=device)
        for b in range(w.B):
            gen = torch.Generator(device=device)
            gen.manual_seed(((w.cfg_id * 1000 + layer_id) * 100 + tag) * 100000 + b)
            n = int(lengths[b]) - 1
            if n > 0:
                g = torch.randn((n, Hk, d_h), generator=gen, device=device,
                                dtype=torch.float32)
                c[b, :n] = _unit_rms(g).to(dt)
            if poison:
                c[b, max(n, 0):] = float("nan")
            else:
                c[b, max(n, 0):] = 0
        caches.append(c)
    return caches[0], caches[1]
