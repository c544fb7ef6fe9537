"""GPU parity of a routed stack of blocks ("Global vs Local Layer Routing",
How it works): layer l has type P[l mod 6] with that type's (theta, scale),
each block's output feeds the next; gemma3_stack_prefill, the variant that
fills one left-aligned cache per layer (gemma3_stack_prefill_cache) and the
stack decode step (gemma3_stack_decode), against the fp64 oracle.

Bars. fp32: 1e-4. bf16: every layer is checked at the block's own bar
(6e-2 + 1e-2 |ref| per element, relative RMS <= 1.5e-2, see the block
tests) by teacher forcing: the type of layer l does not depend on the depth
(P[l mod 6]), so a stack of depth l + 1 is the first l + 1 layers of any
deeper one, and its output is compared with the oracle's block l applied to
the GPU's output at depth l. Each layer's cache is compared the same way
(the oracle's cache fill of the GPU's input to that layer) at the attention
path's bar (2e-2 + 1e-2 |ref|). The whole stack against the oracle's whole
stack is held to the relative-RMS bar (1.5e-2), which an error in any one
layer's structure (a wrong type, rotation or norm) exceeds by far; its
largest element error is logged (about 0.19 on 7 layers, where each layer
adds its own rounding to a residual stream the later layers carry on).
"""

import numpy as np
import pytest
import torch

import workloads as W
from workloads import inputs as I
from parity_util import (REL_RMS_BF16, assert_bf16_close, assert_f32_close, err_stats, f64,
                         log, small_prefill_inputs)
import oracle as O

pytestmark = pytest.mark.gpu

ATTN_KEYS = ("w_q", "w_kv", "w_o", "gamma_q", "gamma_k")
BLOCK_KEYS = ("pre_attn_norm", "post_attn_norm", "pre_ffw_norm", "post_ffw_norm", "w_gating",
              "w_linear")


def _layer_weights(seed, D, H, Hk, d_h, D_ff, dtype):
    r = np.random.default_rng([seed, D, D_ff])
    std = D ** -0.5
    w = dict(w_q=r.standard_normal((H * d_h, D)) * std,
             w_kv=r.standard_normal((2 * Hk * d_h, D)) * std,
             w_o=r.standard_normal((D, H * d_h)) * std,
             gamma_q=r.standard_normal(d_h) * 0.1, gamma_k=r.standard_normal(d_h) * 0.1,
             w_gating=r.standard_normal((2, D_ff, D)) * std,
             w_linear=r.standard_normal((D, D_ff)) * D_ff ** -0.5)
    for k in BLOCK_KEYS[:4]:
        w[k] = r.standard_normal(D) * 0.1
    return {k: I.to_dtype(v, dtype) for k, v in w.items()}


L, G = "LOCAL_SLIDING", "GLOBAL"
ATOL_BLOCK = 6e-2


def _okw(kw):
    return dict(num_heads=kw["H"], num_kv_heads=kw["H_kv"], head_dim=kw["d_h"],
                window=kw["window"], local_rope=kw["local_rope"], global_rope=kw["global_rope"],
                query_scale=kw["query_scale"])


def _routed(l, kw):
    t = O.layer_attn_type(l, l + 1)
    theta, scale = kw["local_rope"] if t == L else kw["global_rope"]
    return dict(attn_type=t, rope_theta=theta, rope_scale=scale)


def _f64w(w):
    return {k: f64(v) for k, v in w.items()}


def assert_block_close(g, r, what, dtype):
    if dtype == "f32":
        assert_f32_close(g, r, what)
        return
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    st = err_stats(g, r)
    log(f"  {what}: {st}")
    bad = np.abs(g - r) > ATOL_BLOCK + 1e-2 * np.abs(r)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside 6e-2 + 1e-2|r|: {st}"
    assert st["rel_rms"] <= REL_RMS_BF16, f"{what}: relative RMS {st['rel_rms']:.3g}"


def _block_ref(h, pos, w, l, kw, lens):
    o = _okw(kw)
    return O.block_prefill(h, pos, w, w["pre_attn_norm"], w["post_attn_norm"], w["pre_ffw_norm"],
                           w["post_ffw_norm"], w["w_gating"], w["w_linear"],
                           num_heads=o["num_heads"], num_kv_heads=o["num_kv_heads"],
                           head_dim=o["head_dim"], window=o["window"],
                           query_scale=o["query_scale"], kv_valid_len=lens, **_routed(l, kw))


def _check(gpu_lib, x, pos, lens, layers, kw, dtype, per_layer=True):
    dev = [{k: v.cuda() for k, v in w.items()} for w in layers]
    xd, pd = x.cuda(), pos.cuda()
    ld = None if lens is None else lens.cuda()
    lens_np = None if lens is None else lens.numpy()
    y = gpu_lib.stack_prefill(xd, pd, dev, kv_valid_len=ld, **kw)
    torch.cuda.synchronize()
    fw = [_f64w(w) for w in layers]
    ref = O.stack_prefill(f64(x), pos.numpy(), fw, kv_valid_len=lens_np, **_okw(kw))
    g = f64(y)
    if dtype == "f32":
        assert_f32_close(g, ref, "stack y")
    else:
        st = err_stats(g, ref)
        log(f"  stack y (whole stack against the whole oracle stack): {st}")
        assert np.all(np.isfinite(g))
        assert st["rel_rms"] <= REL_RMS_BF16, st
    if not per_layer:
        return
    # teacher forcing: layer l against the oracle's block l on the GPU's input
    h = f64(x)
    for l in range(len(layers)):
        yl = y if l == len(layers) - 1 else gpu_lib.stack_prefill(xd, pd, dev[:l + 1],
                                                                  kv_valid_len=ld, **kw)
        torch.cuda.synchronize()
        assert_block_close(f64(yl), _block_ref(h, pos.numpy(), fw[l], l, kw, lens_np),
                           f"layer {l} ({O.layer_attn_type(l, l + 1)})", dtype)
        h = f64(yl)


@pytest.mark.parametrize("dtype,n_layers", [("bf16", 7), ("f32", 7), ("bf16", 1)])
def test_stack_small(gpu_lib, dtype, n_layers):
    B, T, D, H, Hk, d_h, D_ff, Wn = 2, 150, 256, 4, 2, 64, 512, 48
    log(f"stack of {n_layers} {dtype}")
    inp = small_prefill_inputs(71, B, T, D, H, Hk, d_h, dtype, (150, 111))
    layers = [_layer_weights(72 + l, D, H, Hk, d_h, D_ff, dtype) for l in range(n_layers)]
    kw = dict(H=H, H_kv=Hk, d_h=d_h, window=Wn, query_scale=d_h ** -0.5,
              local_rope=(1e4, 1.0), global_rope=(1e6, 8.0))
    _check(gpu_lib, inp["x"], inp["segment_pos"], inp["kv_valid_len"], layers, kw, dtype)


def test_stack_1b_shape_six_layers(gpu_lib):
    # one six-slot tile of 1B-shaped layers (five local with W = 512, one
    # global), T = 4096, D_ff = 6 D; every output compared
    w = W.WORKLOADS[2]
    log("1B-shaped stack of 6")
    x = I.prefill_inputs(w, 0)["x"]
    pos = torch.arange(w.T, dtype=torch.int32).repeat(w.B, 1).contiguous()
    layers = [_layer_weights(80 + l, w.D, w.H, w.H_kv, w.d_h, 6 * w.D, "bf16") for l in range(6)]
    kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, window=w.window, query_scale=w.query_scale,
              local_rope=(1e4, 1.0), global_rope=(1e6, 1.0))
    _check(gpu_lib, x, pos, None, layers, kw, "bf16", per_layer=False)


@pytest.mark.parametrize("dtype,d_h", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_stack_caches_and_decode(gpu_lib, dtype, d_h):
    # A 7-layer stack (five local, one global, one local) fills one cache per
    # layer from tokens 0..T-1 (row 1 padded after 111 tokens), then one
    # stack decode step per row continues at its own position (150 and 111).
    # Every layer's cache slots, its decode output and the slot it writes are
    # checked against the oracle by teacher forcing (each layer's GPU input
    # fed to the oracle), then the whole decode step against the oracle's
    # stack decode on the same cache bytes.
    B, T, H, Hk, D_ff, Wn, S = 2, 150, 4, 2, 512, 48, 200
    D = H * d_h   # the workloads' D >= H d_h (bf16 error of y grows as sqrt(H d_h / D))
    n = 7
    log(f"stack caches and decode {dtype} d_h={d_h}")
    inp = small_prefill_inputs(91, B, T, D, H, Hk, d_h, dtype, (150, 111))
    layers = [_layer_weights(92 + l, D, H, Hk, d_h, D_ff, dtype) for l in range(n)]
    fw = [_f64w(w) for w in layers]
    kw = dict(H=H, H_kv=Hk, d_h=d_h, window=Wn, query_scale=d_h ** -0.5,
              local_rope=(1e4, 1.0), global_rope=(1e6, 8.0))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = [torch.full((B, S, Hk, d_h), float("nan"), dtype=tdt, device="cuda") for _ in range(n)]
    vc = [torch.full_like(c, float("nan")) for c in kc]
    dev = [{k: v.cuda() for k, v in w.items()} for w in layers]
    xd, pd = inp["x"].cuda(), inp["segment_pos"].cuda()
    lens = inp["kv_valid_len"]
    gpu_lib.stack_prefill(xd, pd, dev, kv_valid_len=lens.cuda(), k_caches=kc, v_caches=vc, **kw)
    torch.cuda.synchronize()
    slot_close = assert_bf16_close if dtype == "bf16" else assert_f32_close
    h = f64(inp["x"])
    nan = np.full((B, S, Hk, d_h), np.nan)
    for l in range(n):
        w = fw[l]
        r = _routed(l, kw)
        kr, vr = O.prefill_cache(O.rms_norm(h, w["pre_attn_norm"]), inp["segment_pos"].numpy(),
                                 w["w_kv"], w["gamma_k"], nan, nan, num_kv_heads=Hk, head_dim=d_h,
                                 rope_theta=r["rope_theta"], rope_scale=r["rope_scale"],
                                 kv_valid_len=lens.numpy())
        kg, vg = f64(kc[l]), f64(vc[l])
        for b, nb in enumerate(lens.tolist()):
            slot_close(kg[b, :nb], kr[b, :nb], f"layer {l} row {b} k cache")
            slot_close(vg[b, :nb], vr[b, :nb], f"layer {l} row {b} v cache")
            assert np.all(np.isnan(kg[b, nb:])) and np.all(np.isnan(vg[b, nb:])), \
                f"layer {l} row {b}: slots past the valid tokens were written"
        if l + 1 < n:
            h = f64(gpu_lib.stack_prefill(xd, pd, dev[:l + 1], kv_valid_len=lens.cuda(), **kw))

    # decode: token T of row 0 and token 111 of row 1 (the next positions)
    r = np.random.default_rng([93, d_h])
    xt = I.to_dtype(r.standard_normal((B, 1, D)), dtype)
    pt = lens.clone().to(torch.int32).reshape(B, 1)
    cache_before = [(f64(kc[l]), f64(vc[l])) for l in range(n)]
    h = f64(xt)
    y = None
    for l in range(n):
        # depth l + 1 rewrites slot pos of layers 0..l with the same bits
        y = gpu_lib.stack_decode(xt.cuda(), pt.cuda(), dev[:l + 1], kc[:l + 1], vc[:l + 1], **kw)
        torch.cuda.synchronize()
        w = fw[l]
        o = _okw(kw)
        yr, k_new, v_new = O.block_decode(
            h, pt.numpy(), w, w["pre_attn_norm"], w["post_attn_norm"], w["pre_ffw_norm"],
            w["post_ffw_norm"], w["w_gating"], w["w_linear"], cache_before[l][0],
            cache_before[l][1], num_heads=H, num_kv_heads=Hk, head_dim=d_h, window=Wn,
            query_scale=o["query_scale"], **_routed(l, kw))
        assert_block_close(f64(y), yr, f"decode layer {l} ({O.layer_attn_type(l, l + 1)})", dtype)
        for b, p in enumerate(pt[:, 0].tolist()):
            slot_close(f64(kc[l][b, p]), k_new[b], f"decode layer {l} row {b} k slot")
            slot_close(f64(vc[l][b, p]), v_new[b], f"decode layer {l} row {b} v slot")
            assert torch.isnan(kc[l][b, p + 1:].float()).all(), "slots past the position written"
        h = f64(y)
    ref, _ = O.stack_decode(f64(xt), pt.numpy(), fw, [c[0] for c in cache_before],
                            [c[1] for c in cache_before], **_okw(kw))
    st = err_stats(f64(y), ref)
    log(f"  stack decode y (whole stack): {st}")
    if dtype == "f32":
        assert_f32_close(f64(y), ref, "stack decode y")
    else:
        assert st["rel_rms"] <= REL_RMS_BF16, st


def test_stack_decode_rejects_bad_cache_arrays(gpu_lib):
    # a missing layer cache is refused before anything is enqueued
    B, D, H, Hk, d_h, D_ff, S = 1, 256, 4, 2, 64, 512, 64
    layers = [{k: v.cuda() for k, v in _layer_weights(95 + l, D, H, Hk, d_h, D_ff, "bf16").items()}
              for l in range(2)]
    kw = dict(H=H, H_kv=Hk, d_h=d_h, window=16, query_scale=d_h ** -0.5)
    kc = [torch.zeros((B, S, Hk, d_h), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    x = torch.zeros((B, 1, D), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        gpu_lib.stack_decode(x, p, layers, kc[:1], kc[:1], **kw)
