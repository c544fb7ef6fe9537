"""The allocation-free decode entry point (gemma3_attn_decode_static, for
callers that cannot allocate): through the C ABI, two calls in a row on one
GPU, the second with a smaller input, each against gemma3_attn_decode (the
same kernels with a caller workspace) on copies of the same inputs; bitwise
equal outputs and caches, and the first also within the bf16 bar of the
fp64 oracle (every row of the small call, the shortest row of the
full-length one). A shape whose workspace exceeds the static scratch is refused
with nothing enqueued."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from workloads import inputs as I
from parity_util import assert_bf16_close, f64, layer_kw, log, oracle_kw, to_dev, weights_of

pytestmark = pytest.mark.gpu

CASES = [
    # a 12B-like shape at full cache length (36.5 MiB of scratch), global
    dict(B=16, cache_len=131072, len_range=(1024, 131072), layer=0),
    # then a smaller one, local: fewer rows, a shorter cache
    dict(B=3, cache_len=2048, len_range=(1, 2048), layer=1),
]


def _inputs(c):
    w = W.scaled(W.WORKLOADS[5], B=c["B"], cache_len=c["cache_len"], len_range=c["len_range"])
    lengths = I.decode_lengths(w)
    inp = I.decode_inputs(w, c["layer"], lengths)
    kc, vc = I.decode_cache(w, c["layer"], lengths, device="cuda", poison=True)
    return w, inp, kc, vc


def test_static_decode_matches_workspace_decode(gpu_lib):
    for i, c in enumerate(CASES):
        w, inp, kc, vc = _inputs(c)
        layer = w.layers[c["layer"]]
        log(f"static decode call {i}: B={c['B']} S={c['cache_len']} {layer.attn_type}")
        kw = layer_kw(w, layer)
        d = to_dev(inp)
        kc2, vc2 = kc.clone(), vc.clone()
        kc0, vc0 = kc.clone(), vc.clone()
        y_ws = gpu_lib.decode(d["x"], d["segment_pos"], weights_of(d), kc, vc, **kw)
        y_st = gpu_lib.decode_static(d["x"], d["segment_pos"], weights_of(d), kc2, vc2, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y_ws, y_st), "static decode differs from the workspace decode"
        assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
        assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))
        # and the oracle on the same stored cache bytes: every row of the
        # small call, the shortest row of the full-length one
        lens = inp["segment_pos"][:, 0].tolist()
        rows = range(c["B"]) if c["cache_len"] <= 4096 else [int(np.argmin(lens))]
        for b in rows:
            t = int(inp["segment_pos"][b, 0])
            kb = kc0[b:b + 1, :t + 1].float().cpu().numpy()
            vb = vc0[b:b + 1, :t + 1].float().cpu().numpy()
            r, _, _ = O.decode(f64(inp["x"][b:b + 1]), inp["segment_pos"][b:b + 1].numpy(),
                               f64(inp["w_q"]), f64(inp["w_kv"]), f64(inp["w_o"]),
                               f64(inp["gamma_q"]), f64(inp["gamma_k"]), kb, vb,
                               **oracle_kw(kw))
            assert_bf16_close(f64(y_st[b:b + 1]), r, f"call {i} row {b}")
        del kc, vc, kc2, vc2, kc0, vc0
        torch.cuda.empty_cache()


def test_static_decode_refuses_shapes_beyond_the_scratch(gpu_lib):
    # 27B-shaped rows at full cache length need 300 MiB of workspace; the
    # call returns the scratch error before anything is enqueued (y keeps
    # its bits). The caches are small stand-ins: nothing may read them.
    B, D, H, Hk, d_h, S = 128, 5376, 32, 16, 128, 131072
    desc = gpu_lib.make_desc(B=B, T=1, D=D, H=H, H_kv=Hk, d_h=d_h, attn_type="GLOBAL", window=0,
                             rope_theta=1e6, rope_scale=8.0, query_scale=168 ** -0.5,
                             dtype=torch.bfloat16)
    assert gpu_lib.workspace_bytes(desc, S) > gpu_lib.STATIC_SCRATCH_BYTES
    import ctypes
    y = torch.full((B, 1, D), 7.0, dtype=torch.bfloat16, device="cuda")
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    wts = gpu_lib.Weights(*(buf.data_ptr(),) * 5)
    st = gpu_lib._lib.gemma3_attn_decode_static(
        ctypes.byref(desc), buf.data_ptr(), buf.data_ptr(), ctypes.byref(wts), buf.data_ptr(),
        buf.data_ptr(), S, y.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == 10, gpu_lib.STATUS.get(st, st)
    assert bool((y == 7.0).all())
