"""GPU parity of the prefill chunk against a cache (gemma3_attn_prefill_chunk;
"Gemma 3 Attention Block", How it works: the prefill steps with the Cache
passage's slot = position). The chunk's attention reads the caches in place
(keys row by row, values key-major through transposing LDS reads), and the
caches start NaN-filled, so a read of a slot past the valid keys would show.

A sequence prefilled as a cached first part (gemma3_attn_prefill_cache) and
one or more chunks must give the chunk rows of one prefill over the whole
sequence (fp64 oracle, bf16: 2e-2 + 1e-2 |ref|, fp32: 1e-4) and leave the
cache that prefill would leave; a chunk from an empty cache is bit-identical
to the cache-filling prefill."""

import numpy as np
import pytest
import torch

import workloads as W
from workloads import inputs as I
from parity_util import (assert_bf16_close, assert_f32_close, f64, log, oracle_prefill,
                         small_prefill_inputs, to_dev, weights_of)
import oracle as O

pytestmark = pytest.mark.gpu

L, G = "LOCAL_SLIDING", "GLOBAL"


def _kw(H, Hk, d_h, attn_type, window, alpha=None):
    return dict(H=H, H_kv=Hk, d_h=d_h, attn_type=attn_type, window=window,
                rope_theta=1e4 if attn_type == L else 1e6,
                rope_scale=1.0 if attn_type == L else 8.0,
                query_scale=alpha if alpha is not None else d_h ** -0.5)


def _slice(inp, t0, t1, lens=None):
    d = dict(inp, x=inp["x"][:, t0:t1].contiguous(),
             segment_pos=inp["segment_pos"][:, t0:t1].contiguous(), kv_valid_len=None)
    if lens is not None:
        d["kv_valid_len"] = torch.tensor(lens, dtype=torch.int32)
    return d


def _chunked(gpu_lib, inp, kw, cuts, S, last_lens=None):
    """Prefill tokens [0, cuts[0]) into NaN caches, then chunks [cuts[i], cuts[i+1])."""
    B, N, _ = inp["x"].shape
    Hk, d_h = kw["H_kv"], kw["d_h"]
    dt = inp["x"].dtype
    kc = torch.full((B, S, Hk, d_h), float("nan"), dtype=dt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    first = to_dev(_slice(inp, 0, cuts[0]))
    gpu_lib.prefill(first["x"], first["segment_pos"], weights_of(first), k_cache=kc, v_cache=vc,
                    **kw)
    ys = []
    bounds = list(cuts) + [N]
    for i in range(len(cuts)):
        t0, t1 = bounds[i], bounds[i + 1]
        ch = to_dev(_slice(inp, t0, t1, last_lens if i == len(cuts) - 1 else None))
        ys.append(gpu_lib.prefill_chunk(ch["x"], ch["segment_pos"], weights_of(ch), kc, vc, t0,
                                        kv_valid_len=ch["kv_valid_len"], **kw))
    torch.cuda.synchronize()
    return ys, kc, vc


# B, N, D, H, H_kv, d_h, dtype, cuts (the first is the cached part), valid lengths of the
# last chunk, S
CASES = [
    (2, 500, 512, 4, 2, 128, "bf16", (300,), None, 512),
    (2, 500, 512, 4, 2, 128, "bf16", (130, 333), (167, 40), 520),
    (1, 1257, 1024, 4, 1, 256, "bf16", (1000,), None, 1280),
    (3, 321, 256, 4, 4, 64, "bf16", (1, 64, 200), (121, 1, 77), 321),
    (2, 150, 96, 2, 1, 16, "f32", (70,), (80, 33), 160),
    (1, 128, 256, 4, 1, 64, "f32", (50, 51), None, 128),
    # the 27B-shaped heads (d_h = 128, two query heads per KV head, two row
    # blocks per wave), a chunk of 512 after 1024 cached tokens
    (1, 1536, 5376, 32, 16, 128, "bf16", (1024,), None, 1600),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
@pytest.mark.parametrize("attn_type,window", [(L, 100), (G, 0)])
def test_chunks_equal_one_long_prefill(gpu_lib, case, attn_type, window):
    B, N, D, H, Hk, d_h, dtype, cuts, last_lens, S = case
    log(f"case {case} {attn_type}")
    inp = small_prefill_inputs(43, B, N, D, H, Hk, d_h, dtype)
    kw = _kw(H, Hk, d_h, attn_type, window)
    ys, kc, vc = _chunked(gpu_lib, inp, kw, cuts, S, last_lens)
    full_lens = None if last_lens is None else [cuts[-1] + n for n in last_lens]
    ref_inp = dict(inp, kv_valid_len=None if full_lens is None
                   else torch.tensor(full_lens, dtype=torch.int32))
    check = assert_bf16_close if dtype == "bf16" else assert_f32_close
    bounds = list(cuts) + [N]
    ref = oracle_prefill(ref_inp, kw)
    for i, y in enumerate(ys):
        t0, t1 = bounds[i], bounds[i + 1]
        r = ref[:, t0:t1]
        yg = f64(y)
        if full_lens is not None and attn_type == L:
            # rows left with no allowed key output 0 (the library's choice)
            for b in range(B):
                t = np.arange(t0, t1)
                empty = np.minimum(t, full_lens[b] - 1) < t - window + 1
                assert np.all(yg[b, empty] == 0)
                r[b, empty] = 0
        check(yg, r, f"chunk {i} y")
    nan = np.full(tuple(kc.shape), np.nan)
    kr, vr = O.prefill_cache(f64(inp["x"]), inp["segment_pos"].numpy(), f64(inp["w_kv"]),
                             f64(inp["gamma_k"]), nan, nan, num_kv_heads=Hk, head_dim=d_h,
                             rope_theta=kw["rope_theta"], rope_scale=kw["rope_scale"],
                             kv_valid_len=None if full_lens is None else np.array(full_lens))
    kg, vg = f64(kc), f64(vc)
    m = ~np.isnan(kr)
    assert np.array_equal(np.isnan(kg), ~m) and np.array_equal(np.isnan(vg), ~m), \
        "written slots differ from one long prefill's"
    check(kg[m], kr[m], "k slots")
    check(vg[m], vr[m], "v slots")


@pytest.mark.parametrize("dtype,d_h", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("f32", 32)])
@pytest.mark.parametrize("attn_type,window", [(L, 37), (G, 0)])
def test_chunk_from_empty_cache_is_cache_filling_prefill(gpu_lib, dtype, d_h, attn_type, window):
    B, T, H, Hk, S = 2, 200, 4, 2, 256
    D = H * d_h
    log(f"empty-cache chunk {dtype} d_h={d_h} {attn_type}")
    inp = small_prefill_inputs(44, B, T, D, H, Hk, d_h, dtype, (200, 131))
    kw = _kw(H, Hk, d_h, attn_type, window)
    d = to_dev(inp)
    outs = []
    for chunk in (False, True):
        kc = torch.zeros((B, S, Hk, d_h), dtype=d["x"].dtype, device="cuda")
        vc = torch.zeros_like(kc)
        if chunk:
            y = gpu_lib.prefill_chunk(d["x"], d["segment_pos"], weights_of(d), kc, vc, 0,
                                      kv_valid_len=d["kv_valid_len"], **kw)
        else:
            y = gpu_lib.prefill(d["x"], d["segment_pos"], weights_of(d),
                                kv_valid_len=d["kv_valid_len"], k_cache=kc, v_cache=vc, **kw)
        torch.cuda.synchronize()
        outs.append((y, kc, vc))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("layer_id", [0, 1])
def test_chunk_1b_shape_second_half(gpu_lib, layer_id):
    # the 1B-shaped layers: tokens 0..2047 cached, 2048..4095 as one chunk;
    # 96 sampled rows of the chunk against the oracle
    w = W.WORKLOADS[2]
    layer = w.layers[layer_id]
    log(f"1B-shaped chunk, layer {layer_id} {layer.attn_type}")
    inp = I.prefill_inputs(w, layer_id)
    kw = dict(H=w.H, H_kv=w.H_kv, d_h=w.d_h, attn_type=layer.attn_type, window=w.window,
              rope_theta=layer.rope_theta, rope_scale=layer.rope_scale,
              query_scale=w.query_scale)
    ys, kc, vc = _chunked(gpu_lib, inp, kw, (2048,), w.T)
    rows = np.sort(np.random.default_rng(7).choice(np.arange(2048, w.T), 96, replace=False))
    ref = oracle_prefill(inp, kw, rows=rows)
    assert_bf16_close(f64(ys[0])[:, rows - 2048], ref, "sampled chunk rows")


@pytest.mark.parametrize("d_h", [64, 128, 256])
@pytest.mark.parametrize("attn_type,window", [(L, 90), (G, 0)])
def test_chunk_exact_max_pass_reads_cache(gpu_lib, d_h, attn_type, window):
    # alpha = 1 puts every row's logit bound past the fixed-reference range,
    # so the chunk's attention takes the exact-row-maximum pass, whose key
    # loads also come from the caches (NaN past the valid slots). Against the
    # fp64 oracle such logits are limited by the bf16 storage of q and k, so
    # the reference is the GPU's own one-long prefill with the same alpha
    # (same q, k and v bits; the row arithmetic differs only where the key
    # range of a query tile is split differently): bf16 tolerance.
    B, N, D, H, Hk, S, cut = 2, 300, 512, 4, 2, 320, 170
    inp = small_prefill_inputs(46, B, N, D, H, Hk, d_h, "bf16")
    kw = _kw(H, Hk, d_h, attn_type, window, alpha=1.0)
    log(f"exact-max chunk d_h={d_h} {attn_type}")
    ys, _, _ = _chunked(gpu_lib, inp, kw, (cut,), S)
    d = to_dev(inp)
    y_full = gpu_lib.prefill(d["x"], d["segment_pos"], weights_of(d), **kw)
    torch.cuda.synchronize()
    assert_bf16_close(f64(ys[0]), f64(y_full)[:, cut:], "exact-max chunk y")
