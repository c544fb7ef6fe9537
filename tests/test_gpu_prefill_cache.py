"""GPU parity of the cache-filling prefill (gemma3_attn_prefill_cache;
"Gemma 3 Attention Block", How it works, Cache: the call's keys and values go
into a left-aligned buffer, slot = position).

Each case checks, through the C ABI: the written slots against the fp64
oracle's prefill_cache (bf16: 2e-2 + 1e-2 |ref|, fp32: 1e-4), every other
slot unchanged bit for bit (padding tokens and positions past the cache write
nothing), y bit-identical to the plain prefill, and a GPU decode step on the
GPU-filled cache against a plain oracle prefill of the longer sequence."""

import numpy as np
import pytest
import torch

import workloads as W
from workloads import inputs as I
from parity_util import (assert_bf16_close, assert_f32_close, f64, gpu_prefill, log, oracle_kw,
                         oracle_prefill, small_prefill_inputs, to_dev, weights_of)
import oracle as O

pytestmark = pytest.mark.gpu

L, G = "LOCAL_SLIDING", "GLOBAL"


def _kw(H, Hk, d_h, attn_type, window):
    return dict(H=H, H_kv=Hk, d_h=d_h, attn_type=attn_type, window=window,
                rope_theta=1e4 if attn_type == L else 1e6,
                rope_scale=1.0 if attn_type == L else 8.0, query_scale=d_h ** -0.5)


def _old_cache(B, S, Hk, d_h, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, S, Hk, d_h), generator=g).to(dtype)


def _written(pos, lens, S):
    """[B, S] mask of the slots the call writes (valid token, position in range)."""
    B, T = pos.shape
    m = np.zeros((B, S), dtype=bool)
    for b in range(B):
        for t in range(min(T, lens[b])):
            if 0 <= pos[b, t] < S:
                m[b, pos[b, t]] = True
    return m


def _run_and_check(gpu_lib, inp, kw, S, dtype, seed):
    B, T, _ = inp["x"].shape
    Hk, d_h = kw["H_kv"], kw["d_h"]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc0, vc0 = _old_cache(B, S, Hk, d_h, tdt, seed), _old_cache(B, S, Hk, d_h, tdt, seed + 1)
    d = to_dev(inp)
    kc, vc = kc0.cuda(), vc0.cuda()
    y = gpu_lib.prefill(d["x"], d["segment_pos"], weights_of(d),
                        kv_valid_len=d.get("kv_valid_len"), k_cache=kc, v_cache=vc, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, gpu_prefill(gpu_lib, inp, kw)), "y differs from the plain prefill"
    lens = inp.get("kv_valid_len")
    lens = [T] * B if lens is None else [int(v) for v in lens]
    pos = inp["segment_pos"].numpy()
    m = _written(pos, lens, S)
    kr, vr = O.prefill_cache(f64(inp["x"]), pos, f64(inp["w_kv"]), f64(inp["gamma_k"]),
                             f64(kc0), f64(vc0), num_kv_heads=Hk, head_dim=d_h,
                             rope_theta=kw["rope_theta"], rope_scale=kw["rope_scale"],
                             kv_valid_len=np.array(lens))
    kg, vg = kc.cpu(), vc.cpu()
    mt = torch.from_numpy(m)
    assert torch.equal(kg[~mt], kc0[~mt]) and torch.equal(vg[~mt], vc0[~mt]), \
        "a slot that no valid token maps to was modified"
    check = assert_bf16_close if dtype == "bf16" else assert_f32_close
    check(f64(kg)[m], kr[m], "k slots")
    check(f64(vg)[m], vr[m], "v slots")
    return kc, vc


# B, T, D, H, H_kv, d_h, dtype, valid lengths, first position per row, S
CASES = [
    (2, 300, 256, 4, 2, 64, "bf16", (300, 211), (0, 0), 320),
    (2, 257, 512, 4, 1, 128, "bf16", None, (0, 40), 280),      # row 1 runs past the cache
    (1, 200, 512, 2, 2, 256, "bf16", (150,), (7,), 400),
    (3, 65, 1024, 8, 4, 256, "bf16", (65, 1, 64), (0, 0, 3), 70),
    (1, 128, 256, 4, 1, 64, "f32", None, (0,), 128),
    (2, 70, 96, 2, 1, 16, "f32", (70, 33), (5, 0), 72),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_prefill_cache_parity(gpu_lib, case):
    B, T, D, H, Hk, d_h, dtype, lens, starts, S = case
    log(f"case {case}")
    inp = small_prefill_inputs(37, B, T, D, H, Hk, d_h, dtype, lens)
    inp["segment_pos"] = (inp["segment_pos"] +
                          torch.tensor(starts, dtype=torch.int32)[:, None]).contiguous()
    for t, Wn in ((L, 64), (G, 0)):
        _run_and_check(gpu_lib, inp, _kw(H, Hk, d_h, t, Wn), S, dtype, 5)


@pytest.mark.parametrize("attn_type,window", [(G, 1024), (L, 100)])
@pytest.mark.parametrize("d_h", [128, 256])
def test_gpu_decode_continues_gpu_filled_cache(gpu_lib, attn_type, window, d_h):
    # one padded prefill call fills rows of valid lengths L_b; decoding token
    # L_b of each row at position L_b must give the last row of a plain
    # prefill over that row's tokens 0..L_b
    B, T, H, Hk, S = 2, 190, 4, 2, 256
    D = H * d_h
    lens = (190, 123)
    kw = _kw(H, Hk, d_h, attn_type, window)
    log(f"decode after prefill: {attn_type} W={window} d_h={d_h} lens={lens}")
    full = small_prefill_inputs(38, B, T + 1, D, H, Hk, d_h, "bf16")
    inp = dict(full, x=full["x"][:, :T].contiguous(),
               segment_pos=full["segment_pos"][:, :T].contiguous(),
               kv_valid_len=torch.tensor(lens, dtype=torch.int32))
    kc, vc = _run_and_check(gpu_lib, inp, kw, S, "bf16", 9)
    x_dec = torch.stack([full["x"][b, lens[b]] for b in range(B)])[:, None].contiguous()
    pos_dec = torch.tensor(lens, dtype=torch.int32)[:, None].contiguous()
    d = to_dev(dict(full, x=x_dec, segment_pos=pos_dec))
    y = gpu_lib.decode(d["x"], d["segment_pos"], weights_of(d), kc, vc, **kw)
    torch.cuda.synchronize()
    for b in range(B):
        row = dict(full, x=full["x"][b:b + 1, :lens[b] + 1],
                   segment_pos=full["segment_pos"][b:b + 1, :lens[b] + 1])
        ref = oracle_prefill(row, kw, rows=[lens[b]])
        assert_bf16_close(f64(y[b:b + 1]), ref, f"row {b} decode after prefill")


@pytest.mark.parametrize("layer_id", [0, 1])
def test_prefill_cache_1b_shape(gpu_lib, layer_id):
    # the 1B-shaped layers (T = 4096, d_h = 256, one KV head) into a cache of
    # 4608 slots: every slot compared
    w = W.WORKLOADS[2]
    layer = w.layers[layer_id]
    log(f"1B-shaped layer {layer_id} {layer.attn_type}")
    inp = I.prefill_inputs(w, layer_id)
    kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
              rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
              query_scale=w.query_scale)
    _run_and_check(gpu_lib, inp, kw, w.T + 512, "bf16", 11)
