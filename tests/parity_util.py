"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare them.

Tolerances (elementwise):
  fp32 path: |gpu - oracle| <= 1e-4.
  bf16 path: |gpu - oracle| <= 2e-2 + 1e-2 |oracle|, and in addition the
  relative RMS error over the compared set must stay <= 1.5e-2. The second
  bound comes from the arithmetic: the path rounds x-projections, normalised
  Q/K, V, P and O to bf16 (relative step 2^-8, RMS ~ 2^-8/sqrt(3) ~ 2.3e-3 per
  rounding); a handful of independent roundings per output element add up to
  well under 1e-2 relative RMS, while a wrong mask, head map or rotation moves
  outputs by O(1) relative error.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from workloads import inputs as I

ATOL_BF16, RTOL_BF16, REL_RMS_BF16 = 2e-2, 1e-2, 1.5e-2
ATOL_F32 = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_dev(d: dict, dev="cuda"):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def weights_of(d: dict) -> dict:
    return {k: d[k] for k in ("w_q", "w_kv", "w_o", "gamma_q", "gamma_k")}


def layer_kw(w, layer, **over):
    kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
              rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
              query_scale=w.query_scale)
    kw.update(over)
    return kw


def oracle_kw(kw: dict) -> dict:
    return dict(num_heads=kw["H"], num_kv_heads=kw["H_kv"], head_dim=kw["d_h"],
                attn_type=kw["attn_type"], window=kw["window"], rope_theta=kw["rope_theta"],
                rope_scale=kw["rope_scale"], query_scale=kw["query_scale"])


def gpu_prefill(lib, inp_cpu: dict, kw: dict, workspace=None, stages=None):
    d = to_dev(inp_cpu)
    extra = {} if stages is None else {"stages": stages}
    y = lib.prefill(d["x"], d["segment_pos"], weights_of(d), kv_valid_len=d.get("kv_valid_len"),
                    workspace=workspace, **kw, **extra)
    torch.cuda.synchronize()
    return y


def oracle_prefill(inp_cpu: dict, kw: dict, rows=None, **extra):
    lens = inp_cpu.get("kv_valid_len")
    return O.prefill(f64(inp_cpu["x"]), inp_cpu["segment_pos"].numpy(), f64(inp_cpu["w_q"]),
                     f64(inp_cpu["w_kv"]), f64(inp_cpu["w_o"]), f64(inp_cpu["gamma_q"]),
                     f64(inp_cpu["gamma_k"]),
                     kv_valid_len=None if lens is None else lens.numpy(),
                     query_rows=rows, **oracle_kw(kw), **extra)


def err_stats(g: np.ndarray, r: np.ndarray) -> dict:
    e = np.abs(g - r)
    return dict(max_abs=float(e.max()), max_rel=float((e / np.maximum(np.abs(r), 1e-30)).max()),
                rel_rms=float(np.sqrt(np.mean(e ** 2)) / max(np.sqrt(np.mean(r ** 2)), 1e-30)),
                worst_excess=float((e - (ATOL_BF16 + RTOL_BF16 * np.abs(r))).max()))


def assert_bf16_close(g, r, what="", atol=ATOL_BF16):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    st = err_stats(g, r)
    log(f"  {what}: {st}")
    bad = np.abs(g - r) > atol + RTOL_BF16 * np.abs(r)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside {atol:.3g} + 1e-2|r|: {st}"
    assert st["rel_rms"] <= REL_RMS_BF16, f"{what}: relative RMS {st['rel_rms']:.3g}"
    return st


def assert_f32_close(g, r, what="", atol=ATOL_F32):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    e = float(np.abs(g - r).max())
    log(f"  {what}: max_abs={e:.3g}")
    assert e <= atol, f"{what}: max|err| {e:.3g} > {atol}"
    return e


def small_prefill_inputs(seed, B, T, D, H, Hk, d_h, dtype, lens=None):
    """Seeded inputs for scaled-down parity cases (same distributions as the
    workloads: x ~ N(0,1), weights ~ N(0, D^-1/2), gamma ~ N(0, 0.1))."""
    r = np.random.default_rng([seed, B, T, D, H, Hk, d_h])
    std = D ** -0.5
    d = dict(
        x=I.to_dtype(r.standard_normal((B, T, D)), dtype),
        w_q=I.to_dtype(r.standard_normal((H * d_h, D)) * std, dtype),
        w_kv=I.to_dtype(r.standard_normal((2 * Hk * d_h, D)) * std, dtype),
        w_o=I.to_dtype(r.standard_normal((D, H * d_h)) * std, dtype),
        gamma_q=I.to_dtype(r.standard_normal(d_h) * 0.1, dtype),
        gamma_k=I.to_dtype(r.standard_normal(d_h) * 0.1, dtype),
        segment_pos=torch.arange(T, dtype=torch.int32).repeat(B, 1).contiguous(),
        kv_valid_len=None if lens is None else torch.tensor(lens, dtype=torch.int32),
    )
    return d
