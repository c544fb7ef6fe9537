"""Pins of the fp64 oracle against what the pages and the mathematics fix.

No test here retypes the oracle's formula: each one checks a closed form, an
invariant, a special case that reduces to a library routine (torch's rms_norm
and scaled_dot_product_attention in float64), complex-number rotation, or a
per-element brute force on tiny inputs. Constants come from the page fixture
``tests/golden/page_constants.json``. CPU only.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "page_constants.json")))


def _rand(seed, *shape, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _layer(seed, D, H, Hk, d_h, gamma_std=0.1):
    r = np.random.default_rng(seed)
    return dict(
        w_q=r.standard_normal((H * d_h, D)) * D ** -0.5,
        w_kv=r.standard_normal((2 * Hk * d_h, D)) * D ** -0.5,
        w_o=r.standard_normal((D, H * d_h)) * D ** -0.5,
        gamma_q=r.standard_normal(d_h) * gamma_std,
        gamma_k=r.standard_normal(d_h) * gamma_std,
    )


def _prefill(x, wts, pos=None, **kw):
    B, T, _ = x.shape
    if pos is None:
        pos = np.tile(np.arange(T), (B, 1))
    return O.prefill(x, pos, wts["w_q"], wts["w_kv"], wts["w_o"], wts["gamma_q"],
                     wts["gamma_k"], **kw)


# ---------------------------------------------------------------- constants
def test_constants_match_pages():
    assert O.K_MASK == GOLDEN["k_mask"]["value"]
    assert O.RMS_EPS == GOLDEN["rms_eps"]["value"]
    assert list(O.ATTENTION_PATTERN) == GOLDEN["attention_pattern"]["value"]
    g = GOLDEN["query_scale_27b"]
    assert math.isclose((g["D"] / g["H"]) ** -0.5, g["value"], rel_tol=1e-15)
    assert g["D"] // g["H"] == 168 and g["value"] != 128 ** -0.5


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("n", range(1, 101))
def test_routing_prefix_equals_wrap(n):
    types = O.layer_attn_types(n)
    assert types == [O.layer_attn_type(l, n) for l in range(n)]
    assert types[0] == O.LOCAL_SLIDING
    assert types.count(O.GLOBAL) == n // 6
    assert all(types[l] == O.GLOBAL for l in range(5, n, 6))
    assert all(t == O.LOCAL_SLIDING for t in types[n - n % 6:])


def test_routing_watchouts():
    # a 1-based "every 6th layer" rule would make layer 0 global: it is not
    assert O.layer_attn_type(0, 6) == O.LOCAL_SLIDING
    assert O.layer_attn_type(5, 6) == O.GLOBAL
    t = O.layer_attn_types(26)          # depth not a multiple of 6
    assert t.count(O.GLOBAL) == 4 and t[-2:] == [O.LOCAL_SLIDING] * 2
    with pytest.raises(ValueError):
        O.layer_attn_type(6, 6)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms():
    eps = GOLDEN["rms_eps"]["value"]
    for c in (1e-4, 0.3, -2.0, 1e3):
        v = np.full(8, c)
        np.testing.assert_allclose(O.rms_norm(v, np.zeros(8)), c / math.sqrt(c * c + eps),
                                   rtol=1e-15)
    v = np.array([3.0, 4.0, 0.0, 0.0])       # mean square 25/4, nonzero mean
    np.testing.assert_allclose(O.rms_norm(v, np.zeros(4)), v / math.sqrt(6.25 + eps),
                               rtol=1e-15)
    # gamma = -1 zeroes; gamma = 0 is not a T5-style zero scale
    assert np.all(O.rms_norm(v, -np.ones(4)) == 0)
    assert np.all(O.rms_norm(v, np.zeros(4))[:2] != 0)
    g = np.array([0.5, -0.25, 2.0, 1.0])
    np.testing.assert_allclose(O.rms_norm(v, g), v / math.sqrt(6.25 + eps) * (1 + g),
                               rtol=1e-15)


def test_rmsnorm_matches_torch_rms_norm_per_head():
    x = _rand(1, 2, 5, 3, 16) * np.array([1e-3, 1.0, 50.0])[None, None, :, None]
    g = _rand(2, 16, std=0.1)
    ref = F.rms_norm(torch.from_numpy(x), (16,), weight=torch.from_numpy(1 + g), eps=1e-6)
    np.testing.assert_allclose(O.rms_norm(x, g), ref.numpy(), rtol=1e-13, atol=1e-15)


def test_rmsnorm_scale_invariant_and_per_vector():
    x = _rand(3, 4, 64)
    g = _rand(4, 64, std=0.1)
    y = O.rms_norm(x, g)
    x2 = x.copy()
    x2[1] *= 1000.0                       # only that vector's scale changes
    y2 = O.rms_norm(x2, g)
    np.testing.assert_array_equal(np.delete(y2, 1, 0), np.delete(y, 1, 0))
    # scale invariance up to eps: relative change ~ eps / (2 * mean square)
    ms = np.mean(x[1] ** 2)
    np.testing.assert_allclose(y2[1], y[1] * np.sqrt((ms + 1e-6) / (ms + 1e-12)),
                               rtol=1e-12)
    assert np.max(np.abs(y2[1] / y[1] - 1)) > 1e-8


# ---------------------------------------------------------------- RoPE
def _rope_complex(v, p, theta, scale):
    """Rotation written as complex multiplication of (v_i + j v_{i+h})."""
    h = v.shape[-1] // 2
    z = v[..., :h] + 1j * v[..., h:]
    k = np.arange(h)
    z = z * np.exp(1j * (p / scale) * theta ** (-2.0 * k / v.shape[-1]))
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("theta,scale", [(1e4, 1.0), (1e6, 8.0), (1e6, 1.0)])
def test_rope_complex_form_and_norm(theta, scale):
    v = _rand(5, 7, 32)
    pos = np.array([0, 1, 2, 100, 4095, 32767, 131071])
    r = O.rope(v, pos, theta, scale)
    np.testing.assert_allclose(r, _rope_complex(v, pos[:, None], theta, scale),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(v, axis=-1),
                               rtol=1e-13)
    np.testing.assert_array_equal(r[0], v[0])    # position 0 is the identity


def test_rope_pair0_and_frequency():
    d = 4
    e0 = np.zeros(d); e0[0] = 1.0
    # pair 0 turns by exactly p/scale radians, towards channel d/2
    r = O.rope(e0, np.array(12), 1e4, 8.0)
    np.testing.assert_allclose(r, [math.cos(1.5), 0, math.sin(1.5), 0], atol=1e-15)
    # pair 1 at d_h = 4: frequency theta^(-1/2) = 0.01 for theta = 1e4
    e1 = np.zeros(d); e1[1] = 1.0
    r = O.rope(e1, np.array(50), 1e4, 1.0)
    np.testing.assert_allclose(r, [0, math.cos(0.5), 0, math.sin(0.5)], atol=1e-15)


def test_rope_relative_and_scale():
    q, k = _rand(6, 64), _rand(7, 64)
    for m, n in ((10, 3), (5000, 4999), (131071, 7)):
        a = O.rope(q, np.array(m), 1e4, 1.0) @ O.rope(k, np.array(n), 1e4, 1.0)
        b = O.rope(q, np.array(m - n), 1e4, 1.0) @ k
        assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)
    np.testing.assert_allclose(O.rope(q, np.array(16), 1e6, 8.0),
                               O.rope(q, np.array(2), 1e6, 1.0), rtol=1e-14, atol=1e-15)


def test_norm_before_rope_matters_only_with_gamma():
    x = _rand(8, 3, 32)
    pos = np.array([3, 70, 900])
    z = np.zeros(32)
    np.testing.assert_allclose(O.rope(O.rms_norm(x, z), pos, 1e4, 1.0),
                               O.rms_norm(O.rope(x, pos, 1e4, 1.0), z), rtol=1e-12)
    g = _rand(9, 32, std=0.3)
    a = O.rope(O.rms_norm(x, g), pos, 1e4, 1.0)
    b = O.rms_norm(O.rope(x, pos, 1e4, 1.0), g)
    assert np.max(np.abs(a - b)) > 1e-3
    # the oracle's prefill uses the norm-first order
    B, T, D, H, Hk, d_h = 1, 4, 16, 2, 1, 8
    xx = _rand(10, B, T, D)
    w = _layer(11, D, H, Hk, d_h, gamma_std=0.5)
    _, it = _prefill(xx, w, num_heads=H, num_kv_heads=Hk, head_dim=d_h,
                     attn_type=O.GLOBAL, window=0, rope_theta=1e4, rope_scale=1.0,
                     query_scale=0.3, return_intermediates=True)
    pos = np.arange(T)[None, :, None]
    q_first_norm = O.rope(O.rms_norm(it["q"], w["gamma_q"]), pos, 1e4, 1.0)
    np.testing.assert_allclose(it["q_rope"], q_first_norm, rtol=1e-14)
    assert np.max(np.abs(it["q_rope"] - O.rms_norm(O.rope(it["q"], pos, 1e4, 1.0),
                                                   w["gamma_q"]))) > 1e-3


# ---------------------------------------------------------------- projections
def test_projections_select_columns():
    B, T, D, H, Hk, d_h = 2, 3, 10, 2, 1, 2
    x = _rand(12, B, T, D)
    sel_q = np.zeros((H * d_h, D)); sel_kv = np.zeros((2 * Hk * d_h, D))
    for j, c in enumerate([9, 0, 4, 7]):
        sel_q[j, c] = 1.0
    for j, c in enumerate([1, 2, 3, 5]):
        sel_kv[j, c] = 1.0
    q, k, v = O.project_qkv(x, sel_q, sel_kv, H, Hk, d_h)
    np.testing.assert_array_equal(q.reshape(B, T, -1), x[..., [9, 0, 4, 7]])
    np.testing.assert_array_equal(k.reshape(B, T, -1), x[..., [1, 2]])
    np.testing.assert_array_equal(v.reshape(B, T, -1), x[..., [3, 5]])


# ---------------------------------------------------------------- library reduction
def _torch_reference(x, w, pos, H, Hk, d_h, attn_type, W, theta, scale, alpha, lens=None):
    """Torch float64 composition: linear, rms_norm, complex RoPE, SDPA with a
    boolean mask built from explicit comparisons, linear."""
    B, T, D = x.shape
    G = H // Hk
    X = torch.from_numpy(x)
    q = F.linear(X, torch.from_numpy(w["w_q"])).view(B, T, H, d_h)
    kv = F.linear(X, torch.from_numpy(w["w_kv"]))
    k = kv[..., :Hk * d_h].reshape(B, T, Hk, d_h)
    v = kv[..., Hk * d_h:].reshape(B, T, Hk, d_h)
    q = F.rms_norm(q, (d_h,), weight=torch.from_numpy(1 + w["gamma_q"]), eps=1e-6)
    k = F.rms_norm(k, (d_h,), weight=torch.from_numpy(1 + w["gamma_k"]), eps=1e-6)
    q = torch.from_numpy(_rope_complex(q.numpy(), pos[:, :, None, None], theta, scale))
    k = torch.from_numpy(_rope_complex(k.numpy(), pos[:, :, None, None], theta, scale))
    q = alpha * q
    mask = torch.zeros(B, T, T, dtype=torch.bool)
    for b in range(B):
        L = T if lens is None else lens[b]
        for t in range(T):
            for s in range(T):
                ok = s <= t and s < L
                if attn_type == O.LOCAL_SLIDING:
                    ok = ok and (t - W < s < t + W)
                mask[b, t, s] = ok
    kk = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vv = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(q.permute(0, 2, 1, 3), kk, vv,
                                       attn_mask=mask[:, None], scale=1.0)
    o = o.permute(0, 2, 1, 3).reshape(B, T, H * d_h)
    return F.linear(o, torch.from_numpy(w["w_o"])).numpy()


@pytest.mark.parametrize("attn_type,W,theta,scale,lens", [
    (O.GLOBAL, 0, 1e6, 8.0, None),
    (O.LOCAL_SLIDING, 5, 1e4, 1.0, None),
    (O.LOCAL_SLIDING, 3, 1e4, 1.0, (13, 11)),  # no row left without a key
    (O.GLOBAL, 0, 1e6, 1.0, (13, 6)),
])
def test_prefill_matches_torch_sdpa(attn_type, W, theta, scale, lens):
    B, T, D, H, Hk, d_h = 2, 13, 24, 4, 2, 8
    x = _rand(13, B, T, D)
    w = _layer(14, D, H, Hk, d_h)
    pos = np.tile(np.arange(T), (B, 1))
    y = _prefill(x, w, pos, num_heads=H, num_kv_heads=Hk, head_dim=d_h,
                 attn_type=attn_type, window=W, rope_theta=theta, rope_scale=scale,
                 query_scale=0.37, kv_valid_len=lens, q_block=4)
    ref = _torch_reference(x, w, pos, H, Hk, d_h, attn_type, W, theta, scale, 0.37, lens)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- mask / softmax
def _v_of(it):
    return it["v"]


def _core_kw(**kw):
    d = dict(num_heads=4, num_kv_heads=2, head_dim=8, attn_type=O.LOCAL_SLIDING,
             window=4, rope_theta=1e4, rope_scale=1.0, query_scale=0.25)
    d.update(kw)
    return d


def test_window_at_least_T_equals_global():
    x = _rand(15, 2, 11, 16)
    w = _layer(16, 16, 4, 2, 8)
    g = _prefill(x, w, **_core_kw(attn_type=O.GLOBAL, window=0))
    for W in (11, 12, 1000):
        np.testing.assert_array_equal(_prefill(x, w, **_core_kw(window=W)), g)
    assert np.max(np.abs(_prefill(x, w, **_core_kw(window=10)) - g)) > 1e-6


def test_window_one_returns_own_value():
    x = _rand(17, 2, 9, 16)
    w = _layer(18, 16, 4, 2, 8)
    _, it = _prefill(x, w, return_intermediates=True, **_core_kw(window=1))
    v = np.repeat(it["v"], 2, axis=2)
    np.testing.assert_allclose(it["o"], v, rtol=1e-14)


@pytest.mark.parametrize("attn_type,W,lens", [
    (O.LOCAL_SLIDING, 3, None), (O.LOCAL_SLIDING, 4, (9, 12)),
    (O.GLOBAL, 0, (12, 5)), (O.GLOBAL, 0, None)])
def test_zero_query_scale_gives_window_mean(attn_type, W, lens):
    """alpha = 0 makes every allowed logit 0: o_t is the plain mean of V over
    the allowed keys, computed here from prefix sums over the key index."""
    B, T = 2, 12
    x = _rand(19, B, T, 16)
    w = _layer(20, 16, 4, 2, 8)
    _, it = _prefill(x, w, return_intermediates=True, kv_valid_len=lens,
                     **_core_kw(attn_type=attn_type, window=W, query_scale=0.0))
    v = it["v"]
    csum = np.concatenate([np.zeros((B, 1, 2, 8)), np.cumsum(v, axis=1)], axis=1)
    for b in range(B):
        L = T if lens is None else lens[b]
        for t in range(T):
            lo = max(0, t - W + 1) if attn_type == O.LOCAL_SLIDING else 0
            hi = min(t, L - 1)
            assert hi >= lo
            mean = (csum[b, hi + 1] - csum[b, lo]) / (hi - lo + 1)
            for h in range(4):
                np.testing.assert_allclose(it["o"][b, t, h], mean[h // 2], rtol=1e-12,
                                           atol=1e-14)


def test_two_keys_sigmoid_and_query_scale():
    """Row t = 1 of a global layer sees keys 0 and 1: its weight on key 1 is
    sigmoid(alpha * (<q,k1> - <q,k0>)) with the rotated, normalised vectors."""
    x = _rand(21, 1, 2, 16)
    w = _layer(22, 16, 2, 1, 8)
    for alpha in (0.0, 0.25, 1.7):
        _, it = _prefill(x, w, return_intermediates=True,
                         **_core_kw(num_heads=2, num_kv_heads=1, attn_type=O.GLOBAL,
                                    query_scale=alpha))
        kr, v = it["k_rope"][0, :, 0], it["v"][0, :, 0]
        for h in range(2):
            qr = it["q_rope"][0, 1, h]
            s = 1 / (1 + math.exp(-alpha * (qr @ kr[1] - qr @ kr[0])))
            np.testing.assert_allclose(it["o"][0, 1, h], (1 - s) * v[0] + s * v[1],
                                       rtol=1e-12)
            np.testing.assert_allclose(it["o"][0, 0, h], v[0], rtol=1e-14)


def test_fully_masked_row_is_uniform_over_all_keys():
    """With no allowed key, every logit equals K_MASK, so the softmax is
    uniform over all S keys (the fill-value semantics)."""
    x = _rand(23, 1, 6, 16)
    w = _layer(24, 16, 4, 2, 8)
    _, it = _prefill(x, w, return_intermediates=True, kv_valid_len=(0,),
                     **_core_kw(attn_type=O.GLOBAL))
    for h in range(4):
        np.testing.assert_allclose(it["o"][0, :, h], np.broadcast_to(
            it["v"][0, :, h // 2].mean(axis=0), (6, 8)), rtol=1e-12)


def test_rows_are_convex_combinations():
    x = _rand(25, 2, 10, 16)
    w = _layer(26, 16, 4, 2, 8)
    _, it = _prefill(x, w, return_intermediates=True, **_core_kw(query_scale=2.0))
    v = it["v"]
    for b in range(2):
        for h in range(4):
            vv = v[b, :, h // 2]
            assert np.all(it["o"][b, :, h] <= vv.max(axis=0) + 1e-12)
            assert np.all(it["o"][b, :, h] >= vv.min(axis=0) - 1e-12)


# ---------------------------------------------------------------- GQA
def test_gqa_equals_replicated_heads():
    B, T, D, H, Hk, d_h = 2, 9, 16, 6, 2, 8
    G = H // Hk
    x = _rand(27, B, T, D)
    w = _layer(28, D, H, Hk, d_h)
    y = _prefill(x, w, **_core_kw(num_heads=H, num_kv_heads=Hk, head_dim=d_h))
    wk = w["w_kv"][:Hk * d_h].reshape(Hk, d_h, D)
    wv = w["w_kv"][Hk * d_h:].reshape(Hk, d_h, D)
    rep = dict(w)
    rep["w_kv"] = np.concatenate([np.repeat(wk, G, axis=0).reshape(H * d_h, D),
                                  np.repeat(wv, G, axis=0).reshape(H * d_h, D)])
    y_mha = _prefill(x, rep, **_core_kw(num_heads=H, num_kv_heads=H, head_dim=d_h))
    np.testing.assert_allclose(y, y_mha, rtol=1e-12, atol=1e-14)


def test_gqa_head_map_is_contiguous_groups():
    """alpha = 0 and W = 1: head h returns V of KV head h // G, not h % H_kv."""
    x = _rand(29, 1, 5, 16)
    w = _layer(30, 16, 4, 2, 8)
    _, it = _prefill(x, w, return_intermediates=True,
                     **_core_kw(window=1, query_scale=0.0))
    for h in range(4):
        np.testing.assert_allclose(it["o"][0, :, h], it["v"][0, :, h // 2], rtol=1e-14)
    assert np.max(np.abs(it["o"][0, :, 1] - it["v"][0, :, 1])) > 1e-3


# ---------------------------------------------------------------- brute force
def _brute_force(x, w, H, Hk, d_h, attn_type, W, theta, scale, alpha, lens):
    """Per-element loops with the math module only."""
    B, T, D = len(x), len(x[0]), len(x[0][0])
    G = H // Hk
    half = d_h // 2

    def lin(row, Wm, n):
        return [sum(Wm[j][c] * row[c] for c in range(D)) for j in range(n)]

    def norm_rope(vec, gam, p):
        ms = sum(a * a for a in vec) / d_h
        r = 1.0 / math.sqrt(ms + 1e-6)
        u = [vec[c] * r * (1 + gam[c]) for c in range(d_h)]
        out = [0.0] * d_h
        for i in range(half):
            ang = (p / scale) * theta ** (-2.0 * i / d_h)
            out[i] = u[i] * math.cos(ang) - u[i + half] * math.sin(ang)
            out[i + half] = u[i + half] * math.cos(ang) + u[i] * math.sin(ang)
        return out

    y = [[[0.0] * D for _ in range(T)] for _ in range(B)]
    for b in range(B):
        Q, K, V = [], [], []
        for t in range(T):
            qa = lin(x[b][t], w["w_q"], H * d_h)
            kva = lin(x[b][t], w["w_kv"], 2 * Hk * d_h)
            Q.append([[alpha * z for z in norm_rope(qa[h * d_h:(h + 1) * d_h],
                                                     w["gamma_q"], t)] for h in range(H)])
            K.append([norm_rope(kva[k * d_h:(k + 1) * d_h], w["gamma_k"], t)
                      for k in range(Hk)])
            V.append([kva[(Hk + k) * d_h:(Hk + k + 1) * d_h] for k in range(Hk)])
        for t in range(T):
            o = []
            for h in range(H):
                k = h // G
                keys = [s for s in range(T) if s <= t and s < lens[b] and
                        (attn_type == O.GLOBAL or (s > t - W and s < t + W))]
                lg = [sum(Q[t][h][c] * K[s][k][c] for c in range(d_h)) for s in keys]
                m = max(lg)
                e = [math.exp(a - m) for a in lg]
                z = sum(e)
                o += [sum(e[i] / z * V[s][k][c] for i, s in enumerate(keys))
                      for c in range(d_h)]
            y[b][t] = [sum(w["w_o"][j][c] * o[c] for c in range(H * d_h)) for j in range(D)]
    return np.array(y)


@pytest.mark.parametrize("attn_type,W", [(O.LOCAL_SLIDING, 3), (O.GLOBAL, 0)])
def test_prefill_brute_force(attn_type, W):
    B, T, D, H, Hk, d_h = 2, 6, 5, 4, 2, 4
    x = _rand(31, B, T, D)
    w = _layer(32, D, H, Hk, d_h)
    lens = (6, 4)
    y = _prefill(x, w, num_heads=H, num_kv_heads=Hk, head_dim=d_h, attn_type=attn_type,
                 window=W, rope_theta=1e4, rope_scale=2.0, query_scale=0.6,
                 kv_valid_len=lens)
    bf = _brute_force(x.tolist(), {k: v.tolist() for k, v in w.items()}, H, Hk, d_h,
                      attn_type, W, 1e4, 2.0, 0.6, lens)
    np.testing.assert_allclose(y, bf, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- decode
def _decode_from_prefill(attn_type, W, theta, scale, T=14, t=11):
    B, D, H, Hk, d_h = 2, 16, 4, 2, 8
    x = _rand(33, B, T, D)
    w = _layer(34, D, H, Hk, d_h)
    kw = dict(num_heads=H, num_kv_heads=Hk, head_dim=d_h, attn_type=attn_type,
              window=W, rope_theta=theta, rope_scale=scale, query_scale=0.5)
    y_pf, it = _prefill(x[:, :t + 1], w, return_intermediates=True, **kw)
    S = T + 3
    kc = np.full((B, S, Hk, d_h), np.nan)
    vc = np.full((B, S, Hk, d_h), np.nan)
    kc[:, :t] = it["k_rope"][:, :t]
    vc[:, :t] = it["v"][:, :t]
    pos = np.full((B, 1), t)
    y, k_new, v_new = O.decode(x[:, t:t + 1], pos, w["w_q"], w["w_kv"], w["w_o"],
                               w["gamma_q"], w["gamma_k"], kc, vc, **kw)
    return y, k_new, v_new, y_pf, it, t


@pytest.mark.parametrize("attn_type,W,theta,scale", [
    (O.GLOBAL, 0, 1e6, 8.0), (O.LOCAL_SLIDING, 4, 1e4, 1.0),
    (O.LOCAL_SLIDING, 1, 1e4, 1.0)])
def test_decode_equals_last_prefill_row(attn_type, W, theta, scale):
    y, k_new, v_new, y_pf, it, t = _decode_from_prefill(attn_type, W, theta, scale)
    np.testing.assert_allclose(y[:, 0], y_pf[:, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(k_new, it["k_rope"][:, t], rtol=1e-13)
    np.testing.assert_allclose(v_new, it["v"][:, t], rtol=1e-13)


def test_local_decode_short_history_equals_global():
    y_l = _decode_from_prefill(O.LOCAL_SLIDING, 12, 1e4, 1.0)[0]
    y_g = _decode_from_prefill(O.GLOBAL, 0, 1e4, 1.0)[0]
    np.testing.assert_array_equal(y_l, y_g)
    y_w = _decode_from_prefill(O.LOCAL_SLIDING, 11, 1e4, 1.0)[0]
    assert np.max(np.abs(y_w - y_g)) > 1e-6


# ---------------------------------------------------------------- cache-filling prefill
@pytest.mark.parametrize("attn_type,W", [(O.GLOBAL, 0), (O.LOCAL_SLIDING, 4)])
def test_prefill_cache_then_decode_continues_each_row(attn_type, W):
    # Rows of valid lengths L_b fill a NaN cache from one padded prefill call;
    # decoding token L_b of a row at position L_b must then give the last row
    # of a plain prefill over that row's tokens 0..L_b (the cache is what lets
    # a decode step continue the sequence), and no slot past L_b is touched.
    B, T, D, H, Hk, d_h, S = 3, 12, 16, 4, 2, 8, 20
    lens = np.array([12, 7, 1])
    x = _rand(41, B, T + 1, D)
    w = _layer(42, D, H, Hk, d_h)
    kw = dict(num_heads=H, num_kv_heads=Hk, head_dim=d_h, attn_type=attn_type, window=W,
              rope_theta=1e4, rope_scale=1.0, query_scale=0.4)
    pos = np.tile(np.arange(T), (B, 1))
    nan = np.full((B, S, Hk, d_h), np.nan)
    kc, vc = O.prefill_cache(x[:, :T], pos, w["w_kv"], w["gamma_k"], nan, nan,
                             num_kv_heads=Hk, head_dim=d_h, rope_theta=1e4, rope_scale=1.0,
                             kv_valid_len=lens)
    for b in range(B):
        L = int(lens[b])
        assert not np.isnan(kc[b, :L]).any() and not np.isnan(vc[b, :L]).any()
        assert np.isnan(kc[b, L:]).all() and np.isnan(vc[b, L:]).all()
        y_ref = _prefill(x[b:b + 1, :L + 1], w, **kw)[0, L]
        y, _, _ = O.decode(x[b:b + 1, L:L + 1], np.array([[L]]), w["w_q"], w["w_kv"],
                           w["w_o"], w["gamma_q"], w["gamma_k"], kc[b:b + 1], vc[b:b + 1], **kw)
        np.testing.assert_allclose(y[0, 0], y_ref, rtol=1e-12, atol=1e-14)


def test_prefill_cache_slots_follow_positions():
    # slot = position: a row whose positions start at 5 fills slots 5.. and
    # stops at the end of the cache, a negative position writes nothing, and
    # every other slot keeps its contents
    B, T, D, H, Hk, d_h, S = 2, 6, 16, 2, 2, 8, 9
    x = _rand(43, B, T, D)
    w = _layer(44, D, H, Hk, d_h)
    pos = np.array([[5, 6, 7, 8, 9, 10], [-1, 0, 1, 2, 3, 4]])
    old_k, old_v = _rand(45, B, S, Hk, d_h), _rand(46, B, S, Hk, d_h)
    kc, vc = O.prefill_cache(x, pos, w["w_kv"], w["gamma_k"], old_k, old_v,
                             num_kv_heads=Hk, head_dim=d_h, rope_theta=1e4, rope_scale=2.0)
    _, k, v = O.project_qkv(x, w["w_q"], w["w_kv"], H, Hk, d_h)
    k_rope = O.rope(O.rms_norm(k, w["gamma_k"]), pos[:, :, None], 1e4, 2.0)
    written = {(0, 5): 0, (0, 6): 1, (0, 7): 2, (0, 8): 3,
               (1, 0): 1, (1, 1): 2, (1, 2): 3, (1, 3): 4, (1, 4): 5}
    for b in range(B):
        for s in range(S):
            t = written.get((b, s))
            if t is None:
                np.testing.assert_array_equal(kc[b, s], old_k[b, s])
                np.testing.assert_array_equal(vc[b, s], old_v[b, s])
            else:
                np.testing.assert_allclose(kc[b, s], k_rope[b, t], rtol=1e-13, atol=1e-15)
                np.testing.assert_allclose(vc[b, s], v[b, t], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("attn_type,W,lens", [(O.GLOBAL, 0, None), (O.LOCAL_SLIDING, 4, None),
                                              (O.LOCAL_SLIDING, 6, (7, 3)), (O.GLOBAL, 0, (7, 1))])
def test_prefill_chunk_equals_one_long_prefill(attn_type, W, lens):
    # a sequence of N = start + T tokens prefilled as a cached first part and a
    # chunk gives the chunk's rows of one prefill over all N tokens (the chunk's
    # padding is that prefill's padding), and leaves the cache one prefill of
    # all N tokens would leave
    B, start, T, D, H, Hk, d_h, S = 2, 9, 7, 16, 4, 2, 8, 20
    N = start + T
    x = _rand(47, B, N, D)
    w = _layer(48, D, H, Hk, d_h)
    kw = dict(num_heads=H, num_kv_heads=Hk, head_dim=d_h, attn_type=attn_type, window=W,
              rope_theta=1e4, rope_scale=1.0, query_scale=0.45)
    ck = dict(num_kv_heads=Hk, head_dim=d_h, rope_theta=1e4, rope_scale=1.0)
    pos = np.tile(np.arange(N), (B, 1))
    nan = np.full((B, S, Hk, d_h), np.nan)
    kc, vc = O.prefill_cache(x[:, :start], pos[:, :start], w["w_kv"], w["gamma_k"], nan, nan,
                             **ck)
    y, kc2, vc2 = O.prefill_chunk(x[:, start:], pos[:, start:], w["w_q"], w["w_kv"], w["w_o"],
                                  w["gamma_q"], w["gamma_k"], kc, vc, start, **kw,
                                  kv_valid_len=lens)
    full_lens = None if lens is None else np.array(lens) + start
    y_full = _prefill(x, w, kv_valid_len=full_lens, **kw)
    np.testing.assert_allclose(y, y_full[:, start:], rtol=1e-12, atol=1e-14)
    kf, vf = O.prefill_cache(x, pos, w["w_kv"], w["gamma_k"], nan, nan, kv_valid_len=full_lens,
                             **ck)
    np.testing.assert_array_equal(np.isnan(kc2), np.isnan(kf))
    np.testing.assert_allclose(np.nan_to_num(kc2), np.nan_to_num(kf), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(np.nan_to_num(vc2), np.nan_to_num(vf), rtol=1e-13, atol=1e-15)


def test_prefill_chunk_from_empty_cache_is_plain_prefill():
    B, T, D, H, Hk, d_h = 2, 8, 16, 2, 1, 8
    x = _rand(49, B, T, D)
    w = _layer(50, D, H, Hk, d_h)
    kw = dict(num_heads=H, num_kv_heads=Hk, head_dim=d_h, attn_type=O.LOCAL_SLIDING, window=3,
              rope_theta=1e6, rope_scale=8.0, query_scale=0.3)
    pos = np.tile(np.arange(T), (B, 1))
    zero = np.zeros((B, T, Hk, d_h))
    y, _, _ = O.prefill_chunk(x, pos, w["w_q"], w["w_kv"], w["w_o"], w["gamma_q"],
                              w["gamma_k"], zero, zero, 0, **kw)
    np.testing.assert_allclose(y, _prefill(x, w, **kw), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- full block (GeGLU MLP, norms)
def test_gelu_tanh_against_torch_and_odd_part():
    u = np.linspace(-8, 8, 1601)
    ref = F.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(u), ref, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.gelu_tanh(u) - O.gelu_tanh(-u), u, rtol=1e-14, atol=1e-15)
    assert O.gelu_tanh(0.0) == 0.0


def test_feed_forward_against_torch():
    r = np.random.default_rng(51)
    D, Dff = 24, 40
    u = r.standard_normal((3, 5, D))
    wg = r.standard_normal((2, Dff, D)) * D ** -0.5
    wl = r.standard_normal((D, Dff)) * Dff ** -0.5
    t = torch.from_numpy
    ref = (F.gelu(t(u) @ t(wg[0]).T, approximate="tanh") * (t(u) @ t(wg[1]).T)) @ t(wl).T
    np.testing.assert_allclose(O.feed_forward(u, wg, wl), ref.numpy(), rtol=1e-13, atol=1e-14)


def _block_case(seed, zero_o=False, zero_ffn=False):
    B, T, D, H, Hk, d_h, Dff = 2, 11, 16, 4, 2, 8, 24
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, T, D))
    w = _layer(seed + 1, D, H, Hk, d_h)
    if zero_o:
        w["w_o"] = np.zeros_like(w["w_o"])
    norms = [r.standard_normal(D) * 0.1 for _ in range(4)]
    wg = r.standard_normal((2, Dff, D)) * D ** -0.5
    wl = np.zeros((D, Dff)) if zero_ffn else r.standard_normal((D, Dff)) * Dff ** -0.5
    kw = dict(num_heads=H, num_kv_heads=Hk, head_dim=d_h, attn_type=O.LOCAL_SLIDING, window=4,
              rope_theta=1e4, rope_scale=1.0, query_scale=0.35)
    pos = np.tile(np.arange(T), (B, 1))
    return x, pos, w, norms, wg, wl, kw


def test_block_with_silent_sublayers_is_identity():
    # zero output projection and zero MLP output: both post-norms see zero
    # vectors and give zero, so both residual adds leave x unchanged
    x, pos, w, n, wg, wl, kw = _block_case(52, zero_o=True, zero_ffn=True)
    y = O.block_prefill(x, pos, w, *n, wg, wl, **kw)
    np.testing.assert_array_equal(y, x)


def test_block_post_norm_sits_before_the_residual_add():
    # with gamma_post = 0 each sublayer adds a vector of RMS ~1 over D to the
    # stream (the post-norm output), whatever the stream's own scale
    x, pos, w, n, wg, wl, kw = _block_case(53, zero_ffn=True)
    n = [n[0], np.zeros_like(n[1]), n[2], n[3]]
    for c in (1.0, 100.0):
        y = O.block_prefill(c * x, pos, w, *n, wg, wl, **kw)
        d = y - c * x
        rms = np.sqrt(np.mean(d ** 2, axis=-1))
        np.testing.assert_allclose(rms, 1.0, rtol=1e-4)
    # and the attention sublayer alone is the pinned prefill of the pre-normed stream
    a = _prefill(O.rms_norm(x, n[0]), w, **kw)
    np.testing.assert_allclose(O.block_prefill(x, pos, w, *n, wg, wl, **kw),
                               x + O.rms_norm(a, n[1]), rtol=1e-13, atol=1e-14)


def test_stack_routes_layers_and_chains_blocks():
    # two-layer stack = block(block(x)) with the routed types: layer 0 local,
    # layer 1 local (no global slot in a stack of two); a stack of six ends
    # with a global layer whose (theta, scale) is the global pair
    x, pos, w, n, wg, wl, kw = _block_case(54)
    lay = dict(w, pre_attn_norm=n[0], post_attn_norm=n[1], pre_ffw_norm=n[2], post_ffw_norm=n[3],
               w_gating=wg, w_linear=wl)
    common = dict(num_heads=kw["num_heads"], num_kv_heads=kw["num_kv_heads"],
                  head_dim=kw["head_dim"], window=kw["window"], query_scale=kw["query_scale"])
    bk = dict(kw, rope_theta=1e4, rope_scale=1.0)
    y1 = O.block_prefill(x, pos, w, *n, wg, wl, **bk)
    y2 = O.block_prefill(y1, pos, w, *n, wg, wl, **bk)
    np.testing.assert_array_equal(O.stack_prefill(x, pos, [lay, lay], **common), y2)
    h = x
    for l in range(6):
        t = O.GLOBAL if l == 5 else O.LOCAL_SLIDING
        th, sc = (1e6, 8.0) if t == O.GLOBAL else (1e4, 1.0)
        h = O.block_prefill(h, pos, w, *n, wg, wl, **dict(kw, attn_type=t, rope_theta=th,
                                                        rope_scale=sc))
    np.testing.assert_array_equal(O.stack_prefill(x, pos, [lay] * 6, **common), h)


@pytest.mark.parametrize("attn_type,W", [(O.GLOBAL, 0), (O.LOCAL_SLIDING, 4)])
def test_block_decode_continues_block_prefill(attn_type, W):
    # the cache of a block holds the keys and values of its pre-normed stream:
    # filled from tokens 0..t-1, a block decode step of token t gives the last
    # row of a block prefill over tokens 0..t
    x, pos, w, n, wg, wl, kw = _block_case(55)
    kw = dict(kw, attn_type=attn_type, window=W)
    t, S = 8, 12
    B, _, D = x.shape
    Hk, d_h = kw["num_kv_heads"], kw["head_dim"]
    nan = np.full((B, S, Hk, d_h), np.nan)
    kc, vc = O.prefill_cache(O.rms_norm(x[:, :t], n[0]), pos[:, :t], w["w_kv"], w["gamma_k"],
                             nan, nan, num_kv_heads=Hk, head_dim=d_h,
                             rope_theta=kw["rope_theta"], rope_scale=kw["rope_scale"])
    y, _, _ = O.block_decode(x[:, t:t + 1], np.full((B, 1), t), w, *n, wg, wl, kc, vc, **kw)
    y_ref = O.block_prefill(x[:, :t + 1], pos[:, :t + 1], w, *n, wg, wl, **kw)[:, t]
    np.testing.assert_allclose(y[:, 0], y_ref, rtol=1e-12, atol=1e-13)


def _torch_rms(v, gamma):
    t = torch.from_numpy(np.asarray(v, dtype=np.float64))
    return F.rms_norm(t, (t.shape[-1],), weight=torch.from_numpy(1 + gamma), eps=1e-6)


def _torch_ffn(u, wg, wl):
    t = torch.from_numpy
    return (F.gelu(u @ t(wg[0]).T, approximate="tanh") * (u @ t(wg[1]).T)) @ t(wl).T


def _mlp_branch(h, n, wg, wl):
    """post-FFW RMSNorm of the GeGLU FFN of the pre-FFW-normed stream, all in
    torch float64 (F.rms_norm, F.gelu with the tanh approximation)."""
    return _torch_rms(_torch_ffn(_torch_rms(h, n[2]), wg, wl).numpy(), n[3]).numpy()


def test_block_with_silent_attention_is_residual_plus_mlp_branch():
    # zero output projection: the attention sublayer adds nothing (h = x), so
    # the block is x + RMSNorm_post_ffw(FFN(RMSNorm_pre_ffw(x))), with the
    # four norms' gammas all different (a swapped norm vector fails)
    x, pos, w, n, wg, wl, kw = _block_case(56, zero_o=True)
    y = O.block_prefill(x, pos, w, *n, wg, wl, **kw)
    np.testing.assert_allclose(y, x + _mlp_branch(x, n, wg, wl), rtol=1e-12, atol=1e-13)


def test_block_mlp_branch_has_unit_rms_after_its_post_norm():
    # with gamma_post_ffw = 0 the MLP branch is a unit-RMS vector over D,
    # whatever the scale of the FFN weights or of the stream
    x, pos, w, n, wg, wl, kw = _block_case(57, zero_o=True)
    n = [n[0], n[1], n[2], np.zeros_like(n[3])]
    for c, s in ((1.0, 1.0), (1.0, 1e3), (100.0, 1.0), (100.0, 1e3)):
        y = O.block_prefill(c * x, pos, w, *n, wg, s * wl, **kw)
        rms = np.sqrt(np.mean((y - c * x) ** 2, axis=-1))
        np.testing.assert_allclose(rms, 1.0, rtol=1e-4)


@pytest.mark.parametrize("attn_type,W", [(O.GLOBAL, 0), (O.LOCAL_SLIDING, 3)])
def test_block_mlp_reads_the_stream_after_attention(attn_type, W):
    # With the MLP's output weights zeroed the block returns h = x + a (its
    # post-norm sees zeros); the MLP branch added with real weights must then
    # be exactly the branch evaluated on that h, not on x.
    x, pos, w, n, wg, wl, kw = _block_case(58)
    kw = dict(kw, attn_type=attn_type, window=W)
    h = O.block_prefill(x, pos, w, *n, wg, np.zeros_like(wl), **kw)
    assert np.max(np.abs(h - x)) > 0.1          # the attention does move the stream
    y = O.block_prefill(x, pos, w, *n, wg, wl, **kw)
    np.testing.assert_allclose(y - h, _mlp_branch(h, n, wg, wl), rtol=1e-10, atol=1e-12)
    # invariant form: change token 0 only. Rows t > 0 see it through the
    # attention and no other way, so their MLP branch changes as well when
    # (and only when) some row t > 0 may attend to key 0.
    x2 = x.copy()
    x2[:, 0] += 3.0
    h2 = O.block_prefill(x2, pos, w, *n, wg, np.zeros_like(wl), **kw)
    y2 = O.block_prefill(x2, pos, w, *n, wg, wl, **kw)
    d_branch = np.abs((y2 - h2) - (y - h))[:, 1:]
    reach = np.arange(1, x.shape[1]) < (W if attn_type == O.LOCAL_SLIDING else 10 ** 9)
    assert np.all(d_branch[:, reach].max(axis=-1) > 1e-3)
    assert np.all(d_branch[:, ~reach] == 0)


@pytest.mark.parametrize("attn_type,W", [(O.GLOBAL, 0), (O.LOCAL_SLIDING, 4)])
def test_block_decode_mlp_reads_the_stream_after_attention(attn_type, W):
    # the decode step's MLP branch, likewise, is the branch of h (the step's
    # output with the MLP's output weights zeroed) and the post-norm scales it
    # to unit RMS when its gamma is 0
    x, pos, w, n, wg, wl, kw = _block_case(59)
    kw = dict(kw, attn_type=attn_type, window=W)
    t, S = 7, 10
    B, _, D = x.shape
    Hk, d_h = kw["num_kv_heads"], kw["head_dim"]
    r = np.random.default_rng(60)
    kc = r.standard_normal((B, S, Hk, d_h))
    vc = r.standard_normal((B, S, Hk, d_h))
    xt, pt = x[:, t:t + 1], np.full((B, 1), t)
    h, _, _ = O.block_decode(xt, pt, w, *n, wg, np.zeros_like(wl), kc, vc, **kw)
    assert np.max(np.abs(h - xt)) > 0.1
    y, _, _ = O.block_decode(xt, pt, w, *n, wg, wl, kc, vc, **kw)
    np.testing.assert_allclose(y - h, _mlp_branch(h, n, wg, wl), rtol=1e-10, atol=1e-12)
    n0 = [n[0], n[1], n[2], np.zeros_like(n[3])]
    for s in (1.0, 1e3):
        y, _, _ = O.block_decode(xt, pt, w, *n0, wg, s * wl, kc, vc, **kw)
        h0, _, _ = O.block_decode(xt, pt, w, *n0, wg, np.zeros_like(wl), kc, vc, **kw)
        np.testing.assert_allclose(np.sqrt(np.mean((y - h0) ** 2, axis=-1)), 1.0, rtol=1e-4)


def _stack_case(seed, n_layers):
    B, T, D, H, Hk, d_h, Dff = 2, 10, 16, 4, 2, 8, 24
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, T, D))
    layers = []
    for l in range(n_layers):
        w = _layer(seed + 10 + l, D, H, Hk, d_h)
        w.update(pre_attn_norm=r.standard_normal(D) * 0.1,
                 post_attn_norm=r.standard_normal(D) * 0.1,
                 pre_ffw_norm=r.standard_normal(D) * 0.1,
                 post_ffw_norm=r.standard_normal(D) * 0.1,
                 w_gating=r.standard_normal((2, Dff, D)) * D ** -0.5,
                 w_linear=r.standard_normal((D, Dff)) * Dff ** -0.5)
        layers.append(w)
    kw = dict(num_heads=H, num_kv_heads=Hk, head_dim=d_h, window=3, query_scale=0.35)
    pos = np.tile(np.arange(T), (B, 1))
    return x, pos, layers, kw


def test_stack_decode_continues_stack_prefill():
    # seven layers (five local, one global, one local remainder), window 3:
    # caches filled by a stack prefill of tokens 0..t-1, then a stack decode
    # step of token t, give row t of a stack prefill over tokens 0..t, and
    # every layer's written slot is the slot a longer cache-filling prefill
    # writes
    x, pos, layers, kw = _stack_case(70, 7)
    t, S = 7, 9
    B, _, D = x.shape
    Hk, d_h = kw["num_kv_heads"], kw["head_dim"]
    nan = [np.full((B, S, Hk, d_h), np.nan) for _ in layers]
    _, caches = O.stack_prefill_cache(x[:, :t], pos[:, :t], layers, nan, nan, **kw)
    y, written = O.stack_decode(x[:, t:t + 1], np.full((B, 1), t), layers,
                                [c[0] for c in caches], [c[1] for c in caches], **kw)
    y_ref = O.stack_prefill(x[:, :t + 1], pos[:, :t + 1], layers, **kw)
    np.testing.assert_allclose(y[:, 0], y_ref[:, t], rtol=1e-11, atol=1e-12)
    y_long, long_caches = O.stack_prefill_cache(x[:, :t + 1], pos[:, :t + 1], layers, nan, nan,
                                                **kw)
    np.testing.assert_array_equal(y_long, y_ref)
    for l, ((k_new, v_new), (kc, vc)) in enumerate(zip(written, long_caches)):
        np.testing.assert_allclose(k_new, kc[:, t], rtol=1e-11, atol=1e-12, err_msg=f"layer {l}")
        np.testing.assert_allclose(v_new, vc[:, t], rtol=1e-11, atol=1e-12, err_msg=f"layer {l}")
        assert np.all(np.isnan(kc[:, t + 1:])) and np.all(np.isnan(vc[:, t + 1:]))
        assert not np.any(np.isnan(kc[:, :t + 1]))


def test_stack_caches_hold_each_layers_own_keys():
    # the caches of different layers differ (each holds its own layer's
    # pre-normed stream with its own rotation); a one-layer stack's cache is
    # the cache-filling prefill of that layer's pre-normed input
    x, pos, layers, kw = _stack_case(71, 6)
    B, T, D = x.shape
    Hk, d_h = kw["num_kv_heads"], kw["head_dim"]
    z = [np.zeros((B, T, Hk, d_h)) for _ in layers]
    _, caches = O.stack_prefill_cache(x, pos, layers, z, z, **kw)
    assert np.max(np.abs(caches[0][0] - caches[1][0])) > 0.1
    w = layers[0]
    kc, vc = O.prefill_cache(O.rms_norm(x, w["pre_attn_norm"]), pos, w["w_kv"], w["gamma_k"],
                             z[0], z[0], num_kv_heads=Hk, head_dim=d_h, rope_theta=1e4,
                             rope_scale=1.0)
    _, c1 = O.stack_prefill_cache(x, pos, layers[:1], z, z, **kw)
    np.testing.assert_array_equal(c1[0][0], kc)
    np.testing.assert_array_equal(c1[0][1], vc)
    # the global layer of the six (layer 5) caches the normed keys of its own
    # input (the output of layers 0-4), rotated with the global pair (1e6, 8):
    # unrotated at position 0, the complex-form rotation at position 3
    k0 = O.rms_norm(np.einsum("btd,nd->btn", O.rms_norm(
        O.stack_prefill(x, pos, layers[:5], **kw), layers[5]["pre_attn_norm"]),
        layers[5]["w_kv"][:Hk * d_h]).reshape(B, T, Hk, d_h), layers[5]["gamma_k"])
    np.testing.assert_allclose(caches[5][0][:, 0], k0[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(caches[5][0][:, 3], _rope_complex(k0[:, 3], 3, 1e6, 8.0),
                               rtol=1e-12, atol=1e-13)


def test_kv_cache_footprint_closed_form():
    # 26 layers (the 1B depth: 4 full six-slot tiles + 2 local): 4 global and
    # 22 local layers; 128K slots, one KV head of 256, bf16, batch 1
    per_slot = 2 * 1 * 1 * 256 * 2
    S, W = 131072, 512
    full = O.kv_cache_bytes(26, 1, S, 1, 256, W, 2, False)
    win = O.kv_cache_bytes(26, 1, S, 1, 256, W, 2, True)
    assert full == 26 * S * per_slot
    assert win == (4 * S + 22 * W) * per_slot
    assert O.kv_cache_bytes(5, 1, 100, 1, 256, 512, 2, True) == 5 * 100 * per_slot  # W > S


# ---------------------------------------------------------------- sampled rows
@pytest.mark.parametrize("attn_type,W,lens", [(O.LOCAL_SLIDING, 4, (17, 14)),
                                              (O.GLOBAL, 0, (17, 9))])
def test_sampled_rows_equal_full(attn_type, W, lens):
    B, T, D, H, Hk, d_h = 2, 17, 16, 4, 2, 8
    x = _rand(35, B, T, D)
    w = _layer(36, D, H, Hk, d_h)
    kw = dict(num_heads=H, num_kv_heads=Hk, head_dim=d_h, attn_type=attn_type, window=W,
              rope_theta=1e4, rope_scale=1.0, query_scale=0.4, kv_valid_len=lens)
    full = _prefill(x, w, **kw)
    for rows in ([0], [16], [3, 9, 16], [5, 6, 7, 8]):
        part = _prefill(x, w, query_rows=rows, **kw)
        np.testing.assert_allclose(part, full[:, rows], rtol=1e-12, atol=1e-14)
