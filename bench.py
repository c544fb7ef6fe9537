"""Benchmark of the Gemma 3 attention-block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu] [--no-extra]

A step is one prefill pass of the 27B-shaped pair of layers (one local, one
global; B=1, T=32768, D=5376, H=32, H_kv=16, d_h=128, W=1024, alpha =
168^-1/2, bf16), the largest prefill workload on one GPU, through the C ABI
with inputs resident in HBM. `value` is the whole-call algorithmic TFLOP/s of
that step: 2*M*N*K for the three projections plus 4*d_h*H per allowed
(query, key) pair, never the masked or skipped pairs.

The same run also reports (extra keys, not the headline): the 1B-shaped
pair (B=1, T=4096) and the 4B-like six-layer tile (B=4, T=8192, padded rows)
the same way; the decode step of the 12B-like shape (B=16, D=3840, H=16,
H_kv=8, d_h=256, bf16 cache of 131072 slots, seeded lengths) as a global and
as a local (W=1024) layer in algorithmic GB/s (allowed KV slots, weights, x,
y, cache write) with the 256 MB Infinity Cache flushed between repetitions;
per-kernel times from HIP events on the launch stream; the roofline entry of
the dominant kernel; and the fp64 oracle timed on the host cores on a
bounded sample of the headline workload, as a reported CPU baseline.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = 4                # 27B-shaped local + global pair
EXTRA = (2, 3)              # 1B-shaped pair, 4B-like six-layer tile
CPU_SAMPLE_T = 2048         # oracle sample: the first tokens of the headline workload


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--decode-reps", type=int, default=20)
    p.add_argument("--stage-reps", type=int, default=10)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="headline workload only")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run a plain 512 MiB device copy first (scales the HBM byte counters)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def source_hash(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch of one kernel from the committed counter summary,
    only while every kernel source still matches the one profiled."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    for src, h in rec.get("source_sha256_16", {}).items():
        path = os.path.join(ROOT, src)
        if not os.path.exists(path) or source_hash(path) != h:
            return None
    ent = rec.get("kernels", {}).get(key)
    return None if ent is None else ent.get("bytes_per_launch")


# ------------------------------------------------------------------ work counts
def allowed_pairs(T, attn_type, window, kv_len):
    import numpy as np
    t = np.arange(T)
    hi = np.minimum(t, kv_len - 1)
    lo = np.maximum(0, t - window + 1) if attn_type == "LOCAL_SLIDING" else np.zeros_like(t)
    return int(np.maximum(0, hi - lo + 1).sum())


def stage_flops(w, layer):
    """Algorithmic FLOPs of one layer's three stages."""
    M = w.B * w.T
    lens = w.kv_valid_len() or (w.T,) * w.B
    pairs = sum(allowed_pairs(w.T, layer.attn_type, w.window, L) for L in lens)
    return {"qkv": 2 * M * w.D * (w.H + 2 * w.H_kv) * w.d_h,
            "attention": 4 * w.d_h * w.H * pairs,
            "out": 2 * M * (w.H * w.d_h) * w.D}


def decode_bytes(w, layer, lengths):
    n = [min(int(L), w.window) if layer.attn_type == "LOCAL_SLIDING" else int(L)
         for L in lengths]
    kv = sum(n) * w.H_kv * w.d_h * 2 * 2
    n_qkv = (w.H + 2 * w.H_kv) * w.d_h
    weights = (n_qkv * w.D + w.D * w.H * w.d_h + 2 * w.d_h) * 2
    io = 2 * w.B * w.D * 2 + w.B * w.H_kv * w.d_h * 2 * 2
    return kv, weights + io


# ------------------------------------------------------------------ helpers
def stream_events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


STAGES = (("qkv", "STAGE_QKV_PROJ|STAGE_QK_NORM"), ("attention", "STAGE_ATTN"),
          ("out", "STAGE_OUT_PROJ"))
KERNEL_OF_STAGE = {"qkv": "gemm_bf16_nt (QKV projection, QK-norm/RoPE/alpha epilogue)",
                   "attention": "flash_attn_fwd_bf16 (+ flash_combine when split)",
                   "out": "gemm_bf16_nt (output projection)"}


def bench_prefill(args, torch, W, I, lib, dev, wid, cpu_copy=False):
    """Whole steps (every layer of the workload, in order) and, per layer,
    each stage repeated alone. Returns the summary and, with cpu_copy, the
    CPU tensors of the inputs (for the oracle sample)."""
    w = W.WORKLOADS[wid]
    x_cpu = I.prefill_x(w)
    x = x_cpu.to(dev)
    pos = I.prefill_positions(w).to(dev)
    kvl = I.prefill_kv_valid_len(w)
    kvl = None if kvl is None else kvl.to(dev)
    layers, cpu_w, ws_bytes = [], [], 0
    for li, layer in enumerate(w.layers):
        wc = I.layer_weights(w, li)
        if cpu_copy:
            cpu_w.append(wc)
        kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
                  rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
                  query_scale=w.query_scale)
        desc = lib.make_desc(B=w.B, T=w.T, D=w.D, dtype=torch.bfloat16, **kw)
        ws_bytes = max(ws_bytes, lib.workspace_bytes(desc, 0))
        layers.append(dict(layer=layer, wts={k: v.to(dev) for k, v in wc.items()}, kw=kw,
                           flops=stage_flops(w, layer)))
    # the layers run one after another on one stream and share a workspace
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty((w.B, w.T, w.D), dtype=torch.bfloat16, device=dev)
    step_flops = sum(sum(L["flops"].values()) for L in layers)

    def step():
        for L in layers:
            lib.prefill(x, pos, L["wts"], kv_valid_len=kvl, workspace=ws, y=y, **L["kw"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = stream_events(torch)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    log(f"[{w.name}] step {ms_per_step * 1e3:.1f} us ({wall / args.steps * 1e6:.1f} us wall) "
        f"-> {value:.1f} TFLOP/s ({value / PEAK_BF16_TFLOPS:.1%} of bf16 peak)")

    # per-stage kernel times: events on the launch stream around `stage_reps`
    # back-to-back calls of that stage alone (the workspace holds the earlier
    # stages' results from the full call before). On the bf16 shapes here the
    # projection and QK-norm/RoPE are one kernel (epilogue fusion).
    kernels, seen = [], set()
    for li, L in enumerate(layers):
        key = (L["layer"].attn_type, L["layer"].rope_theta, L["layer"].rope_scale)
        if key in seen:   # repeated layers of a tile have the same shapes and plan
            continue
        seen.add(key)
        lib.prefill(x, pos, L["wts"], kv_valid_len=kvl, workspace=ws, y=y, **L["kw"])
        row = {}
        for name, bits in STAGES:
            st = 0
            for b in bits.split("|"):
                st |= getattr(lib, b)
            a, b_ = stream_events(torch)
            # one untimed call first keeps the GPU busy while the timed ones
            # are enqueued (otherwise the host's first-call latency lands in
            # the timing of the short stages)
            lib.prefill(x, pos, L["wts"], kv_valid_len=kvl, workspace=ws, y=y, stages=st,
                        **L["kw"])
            a.record()
            for _ in range(args.stage_reps):
                lib.prefill(x, pos, L["wts"], kv_valid_len=kvl, workspace=ws, y=y, stages=st,
                            **L["kw"])
            b_.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b_) * 1e3 / args.stage_reps
            tf = L["flops"][name] / (us * 1e-6) / 1e12
            row[name] = us
            kernels.append({"layer": li, "type": L["layer"].attn_type, "stage": name,
                            "kernel": KERNEL_OF_STAGE[name], "us": round(us, 2),
                            "flops": L["flops"][name], "tflops": round(tf, 2),
                            "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        log(f"  layer {li} {L['layer'].attn_type:13s} " +
            " ".join(f"{k}={v:.1f}us" for k, v in row.items()))
    out = {"workload": w.name, "value": round(value, 2), "unit": "TFLOP/s",
           "ms_per_step": round(ms_per_step, 5), "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
           "step_flops": step_flops, "kernels": kernels,
           "config": {"workload": w.name, "B": w.B, "T": w.T, "D": w.D, "H": w.H,
                      "H_kv": w.H_kv, "d_h": w.d_h, "window": w.window,
                      "kv_valid_len": w.kv_valid_len(),
                      "layers": [f"{L['layer'].attn_type}(theta={L['layer'].rope_theta:g},"
                                 f"scale={L['layer'].rope_scale:g})" for L in layers],
                      "step_flops": step_flops, "parallelism": "none (1 GPU)"}}
    del ws, y, x, layers
    torch.cuda.empty_cache()
    return out, (x_cpu, cpu_w)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (got --gpus {args.gpus}); the "
              "multi-GPU sharding is a design note, not an implemented path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from workloads import inputs as I
    from global_layers_amd import lib

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} CUs {props.multi_processor_count}")

    if args.copy_calibration:  # known-size plain copy for the byte counters
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- headline
    head, (x_cpu, cpu_w) = bench_prefill(args, torch, W, I, lib, dev, HEADLINE,
                                         cpu_copy=not args.no_cpu)
    w = W.WORKLOADS[HEADLINE]
    # dominant kernel: the single stage launch with the longest time per step
    dom = max(head["kernels"], key=lambda k: k["us"])
    tkey = f"{w.name}/layer{dom['layer']}/{dom['stage']}"
    roofline = {"kernel": f"{dom['kernel']}, layer {dom['layer']} ({dom['type']})",
                "bound": "mfma", "achieved": dom["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": dom["frac"], "traffic": measured_traffic(tkey),
                "flops_per_launch": dom["flops"], "us_per_launch": dom["us"],
                "launches_per_step": 1}
    attn = [k for k in head["kernels"] if k["stage"] == "attention"]
    attn_tflops = sum(k["flops"] for k in attn) / (sum(k["us"] for k in attn) * 1e-6) / 1e12
    log(f"  dominant kernel {roofline['kernel']}: {dom['tflops']} TFLOP/s "
        f"({dom['frac']:.1%}); attention stages {attn_tflops:.1f} TFLOP/s")

    result = {
        "metric": "prefill attn TFLOP/s (% MFMA bf16 peak); decode KV GB/s (% HBM peak)",
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "frac_of_peak": head["frac_of_peak"],
        "attention_stage_tflops": round(attn_tflops, 2),
        "kernels": head["kernels"],
        "roofline": roofline,
    }

    # ---------------------------------------------------------------- other prefill workloads
    if not args.no_extra:
        extra = {}
        for wid in EXTRA:
            r, _ = bench_prefill(args, torch, W, I, lib, dev, wid)
            extra[r["workload"]] = {k: r[k] for k in ("value", "unit", "ms_per_step",
                                                      "frac_of_peak", "step_flops", "kernels")}
        result["prefill_other"] = extra

    # ---------------------------------------------------------------- decode
    if not args.no_decode:
        result["decode"] = bench_decode(args, torch, np, W, I, lib, dev)
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- CPU baseline
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, x_cpu, cpu_w)

    print(json.dumps(result), flush=True)


def bench_decode(args, torch, np, W, I, lib, dev):
    w = W.WORKLOADS[5]
    lengths = I.decode_lengths(w)
    # Cache flush between repetitions: reading 1 GiB leaves the 256 MB MALL
    # full of clean lines of this buffer, so the timed reads start cold and
    # evict nothing that must be written back first.
    flush = torch.zeros(1 << 27, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    out = {"workload": w.name, "B": w.B, "D": w.D, "H": w.H, "H_kv": w.H_kv, "d_h": w.d_h,
           "cache_slots": w.cache_len, "lengths_sum": int(lengths.sum())}
    for li, layer in enumerate(w.layers):
        name = "global" if layer.attn_type == "GLOBAL" else "local"
        inp = I.decode_inputs(w, li, lengths)
        kc, vc = I.decode_cache(w, li, lengths, device=dev, poison=True)
        xd = inp["x"].to(dev)
        pd = inp["segment_pos"].to(dev)
        wts = {k: inp[k].to(dev) for k in ("w_q", "w_kv", "w_o", "gamma_q", "gamma_k")}
        kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
                  rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
                  query_scale=w.query_scale)
        desc = lib.make_desc(B=w.B, T=1, D=w.D, dtype=torch.bfloat16, **kw)
        ws = lib.new_workspace(desc, w.cache_len, dev)
        y = torch.empty((w.B, 1, w.D), dtype=torch.bfloat16, device=dev)
        kv_bytes, other_bytes = decode_bytes(w, layer, lengths)

        def call(stages=lib.DSTAGE_ALL):
            lib.decode(xd, pd, wts, kc, vc, workspace=ws, y=y, stages=stages, **kw)

        for _ in range(3):
            call()
        times = []
        # the attention stage forms q and the step's k, v (QK-norm, RoPE, alpha,
        # cache write) itself, so it runs without the norm stage
        stage_t = {"qkv_proj": [], "attention": [], "out_proj": []}
        bits = [lib.DSTAGE_QKV_PROJ, lib.DSTAGE_ATTN, lib.DSTAGE_OUT_PROJ]
        for _ in range(args.decode_reps):
            flush.max()
            a, b = stream_events(torch)
            a.record()
            call()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
            # stages one at a time, cache flushed before each
            for bit, key in zip(bits, stage_t):
                flush.max()
                a, b = stream_events(torch)
                a.record()
                call(bit)
                b.record()
                torch.cuda.synchronize()
                stage_t[key].append(a.elapsed_time(b))
        med = float(np.median(times))
        gbs = (kv_bytes + other_bytes) / (med * 1e-3) / 1e9
        st = {k: float(np.median(v)) for k, v in stage_t.items()}
        core_gbs = kv_bytes / (st["attention"] * 1e-3) / 1e9
        out[name] = {
            "ms_median": round(med, 4), "ms_min": round(float(np.min(times)), 4),
            "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "kv_bytes": kv_bytes, "other_bytes": other_bytes,
            "stage_us": {k: round(v * 1e3, 2) for k, v in st.items()},
            "roofline": {"kernel": "decode attention (split-KV partial with QK-norm/RoPE/cache "
                                   "write + combine)",
                         "bound": "hbm", "achieved": round(core_gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(core_gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(f"{w.name}/{name}/attention")},
        }
        log(f"decode {name}: {med * 1e3:.1f} us -> {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%}); "
            f"attention core {core_gbs:.0f} GB/s; stages {out[name]['stage_us']}")
        del kc, vc, ws
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, x_cpu, cpu_w):
    """The fp64 oracle on this host's cores, on a bounded sample of the
    headline workload: its first CPU_SAMPLE_T tokens (the same x rows and
    weights), both layers, so the run stays within about ten seconds."""
    import numpy as np

    import oracle as O
    import workloads as W

    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    ws = W.scaled(w, T=CPU_SAMPLE_T)
    x = x_cpu[:, :CPU_SAMPLE_T].float().numpy().astype(np.float64)
    pos = np.tile(np.arange(CPU_SAMPLE_T), (w.B, 1))
    total, flops = 0.0, 0
    for li, layer in enumerate(w.layers):
        wt = {k: v.float().numpy().astype(np.float64) for k, v in cpu_w[li].items()}
        flops += sum(stage_flops(ws, layer).values())
        t0 = time.perf_counter()
        O.prefill(x, pos, wt["w_q"], wt["w_kv"], wt["w_o"], wt["gamma_q"], wt["gamma_k"],
                  num_heads=w.H, num_kv_heads=w.H_kv, head_dim=w.d_h,
                  attn_type=layer.attn_type, window=w.window, rope_theta=layer.rope_theta,
                  rope_scale=layer.rope_scale, query_scale=w.query_scale)
        total += time.perf_counter() - t0
    value = flops / total / 1e12
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    log(f"cpu baseline (fp64 oracle): {total:.2f} s for {flops:.3g} FLOP -> "
        f"{value * 1e3:.2f} GFLOP/s on {threads} BLAS threads")
    return {"value": round(value, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {CPU_SAMPLE_T} of {w.T} tokens of {w.name} (same inputs), both "
                      f"layers, algorithmic FLOPs of that sample; fp64 numpy, BLAS threads "
                      f"{threads}, affinity {len(os.sched_getaffinity(0))} cores, numpy "
                      f"elementwise ops single-threaded; {cpu_model}",
            "seconds": round(total, 3), "sample_flops": flops}


if __name__ == "__main__":
    main()
