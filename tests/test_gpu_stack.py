"""GPU parity of a routed stack of blocks (gemma3_stack_prefill; "Global vs
Local Layer Routing", How it works): layer l has type P[l mod 6] with that
type's (theta, scale), each block's output feeds the next; against the fp64
oracle's stack_prefill.

Bar: fp32 1e-4. bf16, for L layers: per element 6e-2 L + 1e-2 |ref| (each
block adds at most its own bar of 6e-2 to the residual stream, see the block
tests, and L such errors can add with one sign: the triangle inequality over
the layers), and relative RMS <= 1.5e-2, the same RMS bar as a single layer,
which an error of any one layer's structure (a wrong type, rotation or norm)
exceeds by far. Measured on 7 layers: relative RMS about 1.1e-2, largest
element error about 0.19, where errors adding in quadrature (6e-2 sqrt(7))
would allow only 0.16."""

import numpy as np
import pytest
import torch

import workloads as W
from workloads import inputs as I
from parity_util import REL_RMS_BF16, assert_f32_close, err_stats, f64, log, small_prefill_inputs
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


def _check(gpu_lib, x, pos, lens, layers, kw, dtype):
    dev = [{k: v.cuda() for k, v in w.items()} for w in layers]
    y = gpu_lib.stack_prefill(x.cuda(), pos.cuda(), dev,
                              kv_valid_len=None if lens is None else lens.cuda(), **kw)
    torch.cuda.synchronize()
    ref = O.stack_prefill(f64(x), pos.numpy(), [{k: f64(v) for k, v in w.items()} for w in layers],
                          num_heads=kw["H"], num_kv_heads=kw["H_kv"], head_dim=kw["d_h"],
                          window=kw["window"], local_rope=kw["local_rope"],
                          global_rope=kw["global_rope"], query_scale=kw["query_scale"],
                          kv_valid_len=None if lens is None else lens.numpy())
    g = f64(y)
    if dtype == "f32":
        assert_f32_close(g, ref, "stack y")
        return
    st = err_stats(g, ref)
    log(f"  stack y: {st}")
    atol = 6e-2 * len(layers)
    bad = np.abs(g - ref) > atol + 1e-2 * np.abs(ref)
    assert not bad.any(), f"{int(bad.sum())} elements outside {atol:.3g} + 1e-2|r|: {st}"
    assert st["rel_rms"] <= REL_RMS_BF16, st


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
    _check(gpu_lib, x, pos, None, layers, kw, "bf16")
