"""Layers with H_kv == H and one fused qkv weight ("Gemma 3 Attention Block",
How it works, projections): w_q and w_kv passed as views into a single
[3 H d_h, D] matrix give bit-identical results to separately allocated
copies, for prefill, the cache-filling prefill and decode, and match the fp64
oracle."""

import numpy as np
import pytest
import torch

from parity_util import (assert_bf16_close, f64, log, oracle_prefill, small_prefill_inputs,
                         to_dev)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d_h,H,attn_type,window", [(64, 4, "LOCAL_SLIDING", 64),
                                                     (128, 2, "GLOBAL", 0),
                                                     (256, 4, "GLOBAL", 0)])
def test_fused_qkv_views_equal_separate_weights(gpu_lib, d_h, H, attn_type, window):
    B, T, S = 2, 150, 160
    D = H * d_h
    log(f"fused qkv d_h={d_h} H={H} {attn_type}")
    inp = small_prefill_inputs(41, B, T, D, H, H, d_h, "bf16", (150, 97))
    kw = dict(H=H, H_kv=H, d_h=d_h, attn_type=attn_type, window=window, rope_theta=1e4,
              rope_scale=1.0, query_scale=d_h ** -0.5)
    d = to_dev(inp)
    w_qkv = torch.cat([d["w_q"], d["w_kv"]]).contiguous()
    fused = gpu_lib.fused_qkv_weights(w_qkv, d["w_o"], d["gamma_q"], d["gamma_k"], H=H, d_h=d_h)
    assert fused["w_kv"].data_ptr() == w_qkv.data_ptr() + H * d_h * D * 2
    sep = {k: d[k].clone() for k in ("w_q", "w_kv", "w_o", "gamma_q", "gamma_k")}
    lens = d["kv_valid_len"]
    outs = []
    for w in (fused, sep):
        kc = torch.zeros((B, S, H, d_h), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        y = gpu_lib.prefill(d["x"], d["segment_pos"], w, kv_valid_len=lens, k_cache=kc,
                            v_cache=vc, **kw)
        pos = lens.to(torch.int32)[:, None].contiguous()
        x1 = d["x"][:, :1].contiguous()
        yd = gpu_lib.decode(x1, pos, w, kc, vc, **kw)
        torch.cuda.synchronize()
        outs.append((y, yd, kc, vc))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert_bf16_close(f64(outs[0][0]), oracle_prefill(inp, kw), "y")
