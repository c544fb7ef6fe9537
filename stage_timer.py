"""Per-stage timing of the prefill path on the seeded synthetic workloads.

    python stage_timer.py --workload 4 [--reps 10] [--warmup 3] [--cache] [--block]
    python stage_timer.py --workload 5 [--block]   (decode stages, or whole-block steps)

Every layer of the workload goes through the C ABI one stage at a time
(gemma3_attn_prefill_stages): the projection with its QK-norm / RoPE
epilogue, the attention core, the output projection. Each stage is timed with
HIP events on the call stream over `reps` back-to-back repetitions after
`warmup` untimed ones (so the clocks are at their working level, unlike a
single cold call), and printed in microseconds with its algorithmic TFLOP/s:
projections 2 M K N, attention 4 d_h H per allowed (query, key) pair. With
--cache, the whole layer also runs as gemma3_attn_prefill_cache into a cache
of T slots; the difference to the plain call is the cache fill, printed with
its algorithmic GB/s (each valid token's key and value read once and written
once: 4 H_kv d_h elements). With --block, the layer also runs as a whole
Gemma 3 block (gemma3_block_prefill: norms, attention, GeGLU MLP with
D_ff = 6 D on the 1B shape and 4 D otherwise, seeded synthetic weights), printed
with its algorithmic TFLOP/s (the attention layer's plus 6 M D D_ff for the
MLP). A profiling aid (for example under rocprofv3); the benchmark line is
bench.py's.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from global_layers_amd import lib  # noqa: E402
import workloads as W  # noqa: E402
from workloads import inputs as I  # noqa: E402


def allowed_pairs(T: int, attn_type: str, window: int, kv_len: int) -> int:
    t = np.arange(T)
    hi = np.minimum(t, kv_len - 1)
    lo = np.maximum(0, t - window + 1) if attn_type == W.LOCAL_SLIDING else np.zeros_like(t)
    return int(np.maximum(0, hi - lo + 1).sum())


def stage_flops(w, layer) -> dict:
    M = w.B * w.T
    lens = w.kv_valid_len() or (w.T,) * w.B
    pairs = sum(allowed_pairs(w.T, layer.attn_type, w.window, L) for L in lens)
    return {"qkv": 2 * M * w.D * (w.H + 2 * w.H_kv) * w.d_h,
            "attention": 4 * w.d_h * w.H * pairs,
            "out": 2 * M * w.H * w.d_h * w.D}


def time_layer(w, layer_id: int, reps: int, warmup: int, cache: bool = False) -> dict:
    layer = w.layers[layer_id]
    inp = I.prefill_inputs(w, layer_id)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    weights = {k: d[k] for k in ("w_q", "w_kv", "w_o", "gamma_q", "gamma_k")}
    kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
              rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
              query_scale=w.query_scale)
    B, T, D = d["x"].shape
    desc = lib.make_desc(B=B, T=T, D=D, dtype=d["x"].dtype, **kw)
    ws = lib.new_workspace(desc)
    stream = torch.cuda.current_stream()
    out = {}
    for name, st in (("qkv", lib.STAGE_QKV_PROJ | lib.STAGE_QK_NORM),
                     ("attention", lib.STAGE_ATTN), ("out", lib.STAGE_OUT_PROJ)):
        run = lambda: lib.prefill(d["x"], d["segment_pos"], weights,  # noqa: E731
                                  kv_valid_len=d.get("kv_valid_len"), workspace=ws, stages=st,
                                  **kw)
        for _ in range(warmup):
            run()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / reps
    if cache:
        S = T
        kc = torch.zeros((B, S, w.H_kv, w.d_h), dtype=d["x"].dtype, device="cuda")
        vc = torch.zeros_like(kc)
        for name, extra in (("plain", {}), ("with_cache", dict(k_cache=kc, v_cache=vc))):
            run = lambda: lib.prefill(d["x"], d["segment_pos"], weights,  # noqa: E731
                                      kv_valid_len=d.get("kv_valid_len"), workspace=ws, **extra,
                                      **kw)
            for _ in range(warmup):
                run()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            out[name] = e0.elapsed_time(e1) * 1e3 / reps
    return out


def time_block(w, layer_id: int, reps: int, warmup: int):
    layer = w.layers[layer_id]
    inp = I.prefill_inputs(w, layer_id)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    D = w.D
    D_ff = 6 * D if w.D == 1152 else 4 * D
    g = torch.Generator(device="cuda").manual_seed(1000 + layer_id)
    dt = d["x"].dtype
    for k in ("pre_attn_norm", "post_attn_norm", "pre_ffw_norm", "post_ffw_norm"):
        d[k] = (torch.randn(D, generator=g, device="cuda") * 0.1).to(dt)
    d["w_gating"] = (torch.randn((2, D_ff, D), generator=g, device="cuda") * D ** -0.5).to(dt)
    d["w_linear"] = (torch.randn((D, D_ff), generator=g, device="cuda") * D_ff ** -0.5).to(dt)
    kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
              rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
              query_scale=w.query_scale)
    B, T, _ = d["x"].shape
    desc = lib.make_desc(B=B, T=T, D=D, dtype=dt, **kw)
    ws = torch.empty(lib._lib.gemma3_block_workspace_bytes(ctypes.byref(desc), D_ff),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty_like(d["x"])
    run = lambda: lib.block_prefill(d["x"], d["segment_pos"], d,  # noqa: E731
                                    kv_valid_len=d.get("kv_valid_len"), workspace=ws, y=y, **kw)
    for _ in range(warmup):
        run()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps, 6 * B * T * D * D_ff, D_ff


def time_block_decode(w, layer_id: int, reps: int, warmup: int):
    """A whole-block decode step of the decode workload (D_ff = 4 D): event
    time and the algorithmic bytes (allowed K/V slots, attention and MLP
    weights, each read once)."""
    layer = w.layers[layer_id]
    inp = I.decode_inputs(w, layer_id)
    kc, vc = I.decode_cache(w, layer_id, inp["lengths"], device="cuda", poison=False)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    D = w.D
    D_ff = 4 * D
    g = torch.Generator(device="cuda").manual_seed(2000 + layer_id)
    dt = d["x"].dtype
    for k in ("pre_attn_norm", "post_attn_norm", "pre_ffw_norm", "post_ffw_norm"):
        d[k] = (torch.randn(D, generator=g, device="cuda") * 0.1).to(dt)
    d["w_gating"] = (torch.randn((2, D_ff, D), generator=g, device="cuda") * D ** -0.5).to(dt)
    d["w_linear"] = (torch.randn((D, D_ff), generator=g, device="cuda") * D_ff ** -0.5).to(dt)
    kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
              rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
              query_scale=w.query_scale)
    y = torch.empty_like(d["x"])
    run = lambda: lib.block_decode(d["x"], d["segment_pos"], d, kc, vc, y=y, **kw)  # noqa: E731
    for _ in range(warmup):
        run()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    esz = 2 if dt == torch.bfloat16 else 4
    lens = np.asarray(inp["lengths"])
    slots = np.minimum(lens, w.window) if layer.attn_type == W.LOCAL_SLIDING else lens
    kv = int(slots.sum()) * w.H_kv * w.d_h * 2 * esz
    weights = sum(d[k].numel() for k in ("w_q", "w_kv", "w_o", "w_gating", "w_linear")) * esz
    return e0.elapsed_time(e1) * 1e3 / reps, kv + weights


def time_decode(w, layer_id: int, reps: int, warmup: int) -> dict:
    """The attention decode step of the decode workload stage by stage (the
    projection, split-KV attention with QK-norm/RoPE/cache write, the output
    projection), each stage alone after a 1 GiB read that leaves the 256 MB
    Infinity Cache holding nothing of the step's data; median event time."""
    layer = w.layers[layer_id]
    lengths = I.decode_lengths(w)
    inp = I.decode_inputs(w, layer_id, lengths)
    kc, vc = I.decode_cache(w, layer_id, lengths, device="cuda", poison=True)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    weights = {k: d[k] for k in ("w_q", "w_kv", "w_o", "gamma_q", "gamma_k")}
    kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
              rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
              query_scale=w.query_scale)
    desc = lib.make_desc(B=w.B, T=1, D=w.D, dtype=d["x"].dtype, **kw)
    ws = lib.new_workspace(desc, w.cache_len)
    flush = torch.zeros(1 << 27, dtype=torch.int64, device="cuda")
    out = {}
    for name, st in (("qkv", lib.DSTAGE_QKV_PROJ), ("attention", lib.DSTAGE_ATTN),
                     ("out", lib.DSTAGE_OUT_PROJ), ("step", lib.DSTAGE_ALL)):
        run = lambda: lib.decode(d["x"], d["segment_pos"], weights, kc, vc,  # noqa: E731
                                 workspace=ws, stages=st if name != "step" else lib.DSTAGE_ALL,
                                 **kw)
        if name == "qkv":
            run_all = lambda: lib.decode(d["x"], d["segment_pos"], weights, kc, vc,  # noqa: E731
                                         workspace=ws, **kw)
            for _ in range(warmup):
                run_all()
        ts = []
        for _ in range(reps):
            flush.max()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        out[name] = float(np.median(ts))
    return out


def main() -> None:
    p = argparse.ArgumentParser()
    p.add_argument("--workload", default="4", help="workload ids, comma separated (2, 3, 4)")
    p.add_argument("--reps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cache", action="store_true", help="also time the cache-filling prefill")
    p.add_argument("--block", action="store_true", help="also time the whole Gemma 3 block")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run a plain 512 MiB device copy first (scales the HBM byte counters)")
    args = p.parse_args()
    if not torch.cuda.is_available():
        sys.exit("stage_timer needs a GPU")
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for wid in (int(x) for x in args.workload.split(",")):
        w = W.WORKLOADS[wid]
        if w.T == 1 and not args.block:
            for li, layer in enumerate(w.layers):
                t = time_decode(w, li, args.reps, args.warmup)
                print(f"workload {wid} layer {li} {layer.attn_type:13s} decode " +
                      " | ".join(f"{k} {v:8.1f} us" for k, v in t.items()), flush=True)
            continue
        if w.T == 1:
            for li, layer in enumerate(w.layers):
                us, nbytes = time_block_decode(w, li, args.reps, args.warmup)
                print(f"workload {wid} layer {li} {layer.attn_type:13s} block decode step "
                      f"{us:9.1f} us {nbytes / us / 1e3:8.1f} GB/s "
                      f"({nbytes / 1e6:.0f} MB, {nbytes / us / 1e3 / 8000:.1%} of 8 TB/s)",
                      flush=True)
            continue
        # one layer of each attention type (the others repeat its shapes)
        seen = {}
        for li, layer in enumerate(w.layers):
            seen.setdefault(layer.attn_type, li)
        for attn_type, li in seen.items():
            times = time_layer(w, li, args.reps, args.warmup, args.cache)
            flops = stage_flops(w, w.layers[li])
            parts = [f"{n} {times[n]:9.1f} us {flops[n] / times[n] / 1e6:7.1f} TFLOP/s"
                     for n in ("qkv", "attention", "out")]
            print(f"workload {wid} layer {li} {attn_type:13s} " + " | ".join(parts), flush=True)
            if args.block:
                us, mlp_flops, D_ff = time_block(w, li, args.reps, args.warmup)
                tot = sum(flops.values()) + mlp_flops
                print(f"workload {wid} layer {li} {attn_type:13s} block (D_ff {D_ff}) {us:9.1f} us"
                      f" {tot / us / 1e6:7.1f} TFLOP/s", flush=True)
            if args.cache:
                lens = w.kv_valid_len() or (w.T,) * w.B
                nbytes = 4 * sum(lens) * w.H_kv * w.d_h * (2 if w.dtype == "bf16" else 4)
                dt = times["with_cache"] - times["plain"]
                print(f"workload {wid} layer {li} {attn_type:13s} prefill {times['plain']:9.1f} us"
                      f" | with cache fill {times['with_cache']:9.1f} us | fill {dt:7.1f} us"
                      f" {nbytes / max(dt, 1e-3) / 1e3:7.1f} GB/s ({nbytes / 1e6:.1f} MB)",
                      flush=True)


if __name__ == "__main__":
    main()
