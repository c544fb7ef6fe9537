"""GPU parity of the decode step: HIP path through the C ABI vs the fp64 oracle
on the same seeded inputs and the same stored cache bytes. Slots past each
row's position hold NaN, so any read beyond the allowed range shows up."""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from workloads import inputs as I
from parity_util import (assert_bf16_close, assert_f32_close, f64, layer_kw, log, oracle_kw,
                         to_dev, weights_of)

pytestmark = pytest.mark.gpu


def _run(gpu_lib, w, layer_id, lengths, device="cuda"):
    layer = w.layers[layer_id]
    inp = I.decode_inputs(w, layer_id, lengths)
    kc, vc = I.decode_cache(w, layer_id, lengths, device=device, poison=True)
    kc0, vc0 = kc.clone(), vc.clone()
    kw = layer_kw(w, layer)
    d = to_dev(inp)
    y = gpu_lib.decode(d["x"], d["segment_pos"], weights_of(d), kc, vc, **kw)
    torch.cuda.synchronize()
    return inp, kw, y, kc, vc, kc0, vc0


def _oracle_row(inp, kw, kc, vc, b):
    """Oracle decode of row b from the stored cache bytes (valid prefix only)."""
    t = int(inp["segment_pos"][b, 0])
    kb = kc[b:b + 1, :t + 1].float().cpu().numpy()
    vb = vc[b:b + 1, :t + 1].float().cpu().numpy()
    return O.decode(f64(inp["x"][b:b + 1]), inp["segment_pos"][b:b + 1].numpy(),
                    f64(inp["w_q"]), f64(inp["w_kv"]), f64(inp["w_o"]), f64(inp["gamma_q"]),
                    f64(inp["gamma_k"]), kb, vb, **oracle_kw(kw))


def _check_cache_untouched(kc, vc, kc0, vc0, pos):
    """Only slot pos_b of each row may change."""
    for b, p in enumerate(pos):
        for new, old in ((kc, kc0), (vc, vc0)):
            a, z = new[b], old[b]
            same = (a == z) | (torch.isnan(a) & torch.isnan(z))
            same[p] = True
            assert bool(same.all()), f"row {b}: cache changed outside slot {p}"
            assert not torch.isnan(a[p]).any()


SMALL = [
    # d_h, H, Hk, W, type, lengths, dtype
    (128, 4, 2, 64, "LOCAL_SLIDING", (1, 77, 300), "bf16"),
    (128, 4, 2, 0, "GLOBAL", (1, 77, 300), "bf16"),
    (256, 8, 2, 100, "LOCAL_SLIDING", (250, 2, 99), "bf16"),
    (64, 3, 1, 0, "GLOBAL", (5, 300, 150), "bf16"),
    (256, 2, 2, 0, "GLOBAL", (300, 299, 64), "f32"),
    (64, 4, 1, 16, "LOCAL_SLIDING", (300, 17, 16), "f32"),
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_decode_small(gpu_lib, case):
    d_h, H, Hk, Wn, t, lengths, dtype = case
    log(f"case {case}")
    base = W.WORKLOADS[5]
    w = W.scaled(base, B=len(lengths), D=128, H=H, H_kv=Hk, d_h=d_h, window=max(Wn, 1),
                 query_scale=d_h ** -0.5, cache_len=300, dtype=dtype,
                 layers=(W.Layer(t, 1e6 if t == "GLOBAL" else 1e4, 8.0 if t == "GLOBAL" else 1.0),))
    inp, kw, y, kc, vc, kc0, vc0 = _run(gpu_lib, w, 0, np.array(lengths))
    pos = [int(p) for p in inp["segment_pos"][:, 0]]
    _check_cache_untouched(kc, vc, kc0, vc0, pos)
    for b in range(len(lengths)):
        yr, k_new, v_new = _oracle_row(inp, kw, kc0, vc0, b)
        check = assert_bf16_close if dtype == "bf16" else assert_f32_close
        check(f64(y[b:b + 1]), yr, f"row {b} y")
        check(f64(kc[b, pos[b]]), k_new[0], f"row {b} k slot")
        check(f64(vc[b, pos[b]]), v_new[0], f"row {b} v slot")


@pytest.mark.slow
@pytest.mark.parametrize("layer_id", [0, 1], ids=["global", "local"])
def test_cfg5_full_size_every_row(gpu_lib, layer_id):
    w = W.WORKLOADS[5]
    lengths = I.decode_lengths(w)
    log(f"cfg5 layer {layer_id} lengths {lengths.tolist()}")
    inp, kw, y, kc, vc, kc0, vc0 = _run(gpu_lib, w, layer_id, lengths)
    pos = lengths - 1
    for b in range(w.B):  # every row's written slot and its neighbours
        p = int(pos[b])
        assert torch.isnan(kc[b, p + 1:p + 3].float()).all() or p + 1 >= w.cache_len
    for b in range(w.B):  # every row against the oracle
        log(f"  row {b} length {lengths[b]}")
        yr, k_new, v_new = _oracle_row(inp, kw, kc0, vc0, b)
        assert_bf16_close(f64(y[b:b + 1]), yr, f"row {b} y")
        assert_bf16_close(f64(kc[b, pos[b]]), k_new[0], f"row {b} k slot")
        assert_bf16_close(f64(vc[b, pos[b]]), v_new[0], f"row {b} v slot")
    del kc, vc, kc0, vc0
    torch.cuda.empty_cache()


def test_decode_position_outside_cache_outputs_zero(gpu_lib):
    """A decode position outside [0, S) makes that row skip its cache write and
    output 0 (the documented precondition breach); the other rows are
    unaffected and match the oracle."""
    d_h, H, Hk, Wn, t = 128, 4, 2, 64, "LOCAL_SLIDING"
    lengths = np.array([40, 120, 300, 7])
    base = W.WORKLOADS[5]
    w = W.scaled(base, B=len(lengths), D=128, H=H, H_kv=Hk, d_h=d_h, window=Wn,
                 query_scale=d_h ** -0.5, cache_len=300, dtype="bf16",
                 layers=(W.Layer(t, 1e4, 1.0),))
    inp = I.decode_inputs(w, 0, lengths)
    bad = {1: 300, 3: -1}  # S and -1
    for b, p in bad.items():
        inp["segment_pos"][b, 0] = p
    kc, vc = I.decode_cache(w, 0, lengths, device="cuda", poison=True)
    kc0, vc0 = kc.clone(), vc.clone()
    kw = layer_kw(w, w.layers[0])
    d = to_dev(inp)
    y = gpu_lib.decode(d["x"], d["segment_pos"], weights_of(d), kc, vc, **kw)
    torch.cuda.synchronize()
    for b in range(len(lengths)):
        if b in bad:
            assert torch.all(y[b] == 0), f"row {b}"
            same = (kc[b] == kc0[b]) | (torch.isnan(kc[b]) & torch.isnan(kc0[b]))
            assert bool(same.all()), f"row {b}: k cache written"
            same = (vc[b] == vc0[b]) | (torch.isnan(vc[b]) & torch.isnan(vc0[b]))
            assert bool(same.all()), f"row {b}: v cache written"
        else:
            yr, k_new, _ = _oracle_row(inp, kw, kc0, vc0, b)
            assert_bf16_close(f64(y[b:b + 1]), yr, f"row {b} y")
            assert_bf16_close(f64(kc[b, int(inp["segment_pos"][b, 0])]), k_new[0], f"row {b} k")
