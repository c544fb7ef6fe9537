"""Plain fp64 CPU oracle of the Gemma 3 attention-block forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.

Sources (the study-note pages on Gemma 3):
  * "Gemma 3 Attention Block", How it works: projections, QK-norm -> RoPE ->
    query scale, left-aligned cache, the scores sum, GQA reshape, sliding mask,
    K_MASK fill, softmax, PV, attn_vec_einsum, routing of (theta, scale).
  * "QK-Norm", How it works: the RMSNorm equation with (1 + gamma) and
    eps = 1e-6 over the last axis; norm before RoPE; scale after RoPE; V is
    left alone.
  * "Global vs Local Layer Routing", How it works: the six-slot pattern tiled
    over depth with a prefix remainder; per-type (theta, scale).

Everything is computed in float64. Inputs of any float dtype are read as their
exact values (bf16 and fp32 are exactly representable in fp64). The method is
exact (no approximation), so this module is the definition written out; tiled,
online or split-KV evaluation on the GPU reaches the same result up to rounding.

Readings where the pages leave a step open (each listed with its reason in the
project's design notes):
  * RoPE pairs channel i with channel i + d_h/2 ("half-split"), with angle
    (p / scale) * theta^(-2i/d_h). The pages name RoPE and its (theta, scale)
    pair but never write its formula; the pair layout is therefore a chosen
    convention and is parity-unpinned against the pages.
  * The RoPE scale divides the position (it is described as a positional
    interpolation factor).
  * gamma_Q and gamma_K are vectors of length d_h shared by all heads,
    positions and batch rows.
  * Query head h reads KV head h // G (the [.., H_kv, G, d_h] reshape).
  * Prefill masks are written in token indices t, s; in decode slot s holds
    position s (left-aligned) and the query sits at segment_pos.
  * Weights are stored output-major: w_q [H*d_h, D], w_kv [2*H_kv*d_h, D]
    (K heads first, then V heads), w_o [D, H*d_h]; so Q = x @ w_q.T.
"""

from __future__ import annotations

import numpy as np

# Fill value for blocked logits ("Gemma 3 Attention Block", How it works, Scores).
K_MASK = -2.3819763e38
# RMSNorm epsilon ("QK-Norm", How it works, RMSNorm equation).
RMS_EPS = 1e-6

# AttentionType values ("Global vs Local Layer Routing", How it works).
LOCAL_SLIDING = "LOCAL_SLIDING"
GLOBAL = "GLOBAL"
# Six-slot tile that starts local: (L, L, L, L, L, G).
ATTENTION_PATTERN = (LOCAL_SLIDING,) * 5 + (GLOBAL,)


# --------------------------------------------------------------------------
# Routing ("Global vs Local Layer Routing", How it works)
# --------------------------------------------------------------------------
def layer_attn_type(layer: int, num_layers: int) -> str:
    """type(l) = P[l mod |P|] for l = 0..N-1 (closed form on the routing page)."""
    if not 0 <= layer < num_layers:
        raise ValueError(f"layer {layer} out of range for depth {num_layers}")
    return ATTENTION_PATTERN[layer % len(ATTENTION_PATTERN)]


def layer_attn_types(num_layers: int) -> list:
    """Whole-depth list built the way the routing page says the official config
    does it: the pattern repeated, then a prefix pattern[:N % 6] for the rest."""
    p = list(ATTENTION_PATTERN)
    full, rem = divmod(num_layers, len(p))
    return p * full + p[:rem]


# --------------------------------------------------------------------------
# QK-norm ("QK-Norm", How it works: RMSNorm equation)
# --------------------------------------------------------------------------
def rms_norm(v, gamma, eps: float = RMS_EPS):
    """v / sqrt(mean(v^2 over the last axis) + eps) * (1 + gamma). No centring."""
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * (1.0 + g)


# --------------------------------------------------------------------------
# RoPE ("Gemma 3 Attention Block", How it works; routing page for theta/scale)
# --------------------------------------------------------------------------
def rope(v, pos, theta: float, scale: float):
    """Rotate each (i, i + d_h/2) channel pair by (pos / scale) * theta^(-2i/d_h).

    v: [..., d_h]; pos: broadcastable to v.shape[:-1] (integer positions).
    """
    v = np.asarray(v, dtype=np.float64)
    d_h = v.shape[-1]
    if d_h % 2:
        raise ValueError("RoPE needs an even head dimension")
    half = d_h // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / d_h)
    p = np.asarray(pos, dtype=np.float64) / scale
    phi = p[..., None] * inv_freq
    c, s = np.cos(phi), np.sin(phi)
    x1, x2 = v[..., :half], v[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# --------------------------------------------------------------------------
# Projections ("Gemma 3 Attention Block", How it works: q_einsum / kv_einsum)
# --------------------------------------------------------------------------
def project_qkv(x, w_q, w_kv, num_heads: int, num_kv_heads: int, head_dim: int):
    """Q [B,T,H,d_h], K and V [B,T,H_kv,d_h] from x [B,T,D]."""
    x = np.asarray(x, dtype=np.float64)
    w_q = np.asarray(w_q, dtype=np.float64)
    w_kv = np.asarray(w_kv, dtype=np.float64)
    B, T, _ = x.shape
    q = (x @ w_q.T).reshape(B, T, num_heads, head_dim)
    kv = x @ w_kv.T
    n_k = num_kv_heads * head_dim
    k = kv[..., :n_k].reshape(B, T, num_kv_heads, head_dim)
    v = kv[..., n_k:].reshape(B, T, num_kv_heads, head_dim)
    return q, k, v


# --------------------------------------------------------------------------
# Mask ("Gemma 3 Attention Block", How it works: sliding-mask equation)
# --------------------------------------------------------------------------
def allowed_mask(t_idx, s_idx, attn_type: str, window: int, kv_len):
    """Boolean [len(t_idx), len(s_idx)]: causal, key padding, and on local layers
    the sliding mask 1[s > t - W] * 1[s < t + W]."""
    t = np.asarray(t_idx)[:, None]
    s = np.asarray(s_idx)[None, :]
    ok = (s <= t) & (s < kv_len)
    if attn_type == LOCAL_SLIDING:
        ok &= (s > t - window) & (s < t + window)
    elif attn_type != GLOBAL:
        raise ValueError(f"unknown attention type {attn_type!r}")
    return ok


def attention_core(q, k, v, allowed):
    """One KV head and the query heads of its group.

    q: [Tq, G, d_h] (already normalised, rotated and scaled), k, v: [S, d_h],
    allowed: [Tq, S]. Blocked logits are filled with K_MASK, then a softmax over
    s weights the rows of V. Returns o [Tq, G, d_h].
    """
    Tq, G, d_h = q.shape
    logits = (q.reshape(Tq * G, d_h) @ k.T).reshape(Tq, G, -1)   # sum over c
    logits = np.where(allowed[:, None, :], logits, K_MASK)
    m = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - m)
    p = e / np.sum(e, axis=-1, keepdims=True)
    return (p.reshape(Tq * G, -1) @ v).reshape(Tq, G, d_h)        # sum over s


# --------------------------------------------------------------------------
# Prefill (the whole attention block, no cache)
# --------------------------------------------------------------------------
def prefill(x, segment_pos, w_q, w_kv, w_o, gamma_q, gamma_k, *,
            num_heads: int, num_kv_heads: int, head_dim: int,
            attn_type: str, window: int, rope_theta: float, rope_scale: float,
            query_scale: float, kv_valid_len=None, return_intermediates=False,
            q_block: int = 512, query_rows=None):
    """y [B,T,D] of one attention layer; optionally the intermediates.

    Order: projections -> RMSNorm_Q / RMSNorm_K -> RoPE -> query scale ->
    grouped scores -> mask with K_MASK fill -> softmax -> PV -> output
    projection ("Gemma 3 Attention Block" and "QK-Norm", How it works).

    query_rows: optional sorted token indices; then only those rows of y are
    computed (y is [B, len(query_rows), D]) and keys are projected only over
    the index range some selected row may see. Exact whenever every selected
    row has at least one allowed key (a row with none would average V over
    all T keys, which this mode does not reproduce).
    """
    if query_rows is not None:
        return _prefill_rows(x, segment_pos, w_q, w_kv, w_o, gamma_q, gamma_k,
                             np.asarray(query_rows), num_heads, num_kv_heads, head_dim,
                             attn_type, window, rope_theta, rope_scale, query_scale,
                             kv_valid_len)
    x = np.asarray(x, dtype=np.float64)
    B, T, _ = x.shape
    H, Hk, d_h = num_heads, num_kv_heads, head_dim
    if H % Hk:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = H // Hk
    pos = np.asarray(segment_pos, dtype=np.int64).reshape(B, T)
    lens = (np.full(B, T, dtype=np.int64) if kv_valid_len is None
            else np.asarray(kv_valid_len, dtype=np.int64).reshape(B))

    q, k, v = project_qkv(x, w_q, w_kv, H, Hk, d_h)
    q_hat = rms_norm(q, gamma_q)
    k_hat = rms_norm(k, gamma_k)
    q_rope = rope(q_hat, pos[:, :, None], rope_theta, rope_scale)
    k_rope = rope(k_hat, pos[:, :, None], rope_theta, rope_scale)
    q_tilde = query_scale * q_rope

    o = np.empty((B, T, H, d_h), dtype=np.float64)
    s_idx = np.arange(T)
    for b in range(B):
        for kh in range(Hk):
            kb = k_rope[b, :, kh, :]
            vb = v[b, :, kh, :]
            for t0 in range(0, T, q_block):
                t_idx = np.arange(t0, min(T, t0 + q_block))
                ok = allowed_mask(t_idx, s_idx, attn_type, window, lens[b])
                qb = q_tilde[b, t_idx, kh * G:(kh + 1) * G, :]
                o[b, t_idx, kh * G:(kh + 1) * G, :] = attention_core(qb, kb, vb, ok)

    y = o.reshape(B, T, H * d_h) @ np.asarray(w_o, dtype=np.float64).T
    if not return_intermediates:
        return y
    return y, dict(q=q, k=k, v=v, q_hat=q_hat, k_hat=k_hat, q_rope=q_rope,
                   k_rope=k_rope, q_tilde=q_tilde, o=o)


def prefill_cache(x, segment_pos, w_kv, gamma_k, k_cache, v_cache, *,
                  num_kv_heads: int, head_dim: int, rope_theta: float, rope_scale: float,
                  kv_valid_len=None):
    """Caches after a prefill that fills a left-aligned cache.

    "Gemma 3 Attention Block", How it works, Cache: the call's keys (after
    RMSNorm_K and RoPE) and values are written into a left-aligned buffer of
    S slots, slot = position. Readings: token t of row b goes to slot
    segment_pos[b, t]; tokens at or past kv_valid_len[b] (padding) and
    positions outside [0, S) write nothing; every other slot keeps its
    contents. Returns fp64 copies of k_cache and v_cache [B,S,H_kv,d_h].
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, _ = x.shape
    Hk, d_h = num_kv_heads, head_dim
    w_kv = np.asarray(w_kv, dtype=np.float64)
    k = (x @ w_kv[:Hk * d_h].T).reshape(B, T, Hk, d_h)   # K heads first in w_kv
    v = (x @ w_kv[Hk * d_h:].T).reshape(B, T, Hk, d_h)
    pos = np.asarray(segment_pos, dtype=np.int64).reshape(B, T)
    k_rope = rope(rms_norm(k, gamma_k), pos[:, :, None], rope_theta, rope_scale)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    S = kc.shape[1]
    lens = (np.full(B, T, dtype=np.int64) if kv_valid_len is None
            else np.asarray(kv_valid_len, dtype=np.int64).reshape(B))
    for b in range(B):
        for t in range(min(int(lens[b]), T)):
            p = int(pos[b, t])
            if 0 <= p < S:
                kc[b, p] = k_rope[b, t]
                vc[b, p] = v[b, t]
    return kc, vc


def prefill_chunk(x, segment_pos, w_q, w_kv, w_o, gamma_q, gamma_k, k_cache, v_cache,
                  start: int, *, num_heads: int, num_kv_heads: int, head_dim: int,
                  attn_type: str, window: int, rope_theta: float, rope_scale: float,
                  query_scale: float, kv_valid_len=None):
    """A prefill chunk that continues rows whose first `start` tokens are cached.

    "Gemma 3 Attention Block", How it works, Cache (with the prefill steps of
    the same section): the chunk's T tokens have indices start .. start+T-1;
    their rotated keys and values join the cached slots 0..start-1
    (slot = position) and every query attends under the same masks as a
    prefill of the whole sequence, in those absolute indices. Readings:
    segment_pos[b, t] = start + t feeds RoPE and names the slot the token is
    written to; kv_valid_len[b] counts the chunk's valid tokens (keys past
    start + kv_valid_len[b] are blocked and not written). Returns y [B,T,D]
    and the updated fp64 caches.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, _ = x.shape
    H, Hk, d_h = num_heads, num_kv_heads, head_dim
    G = H // Hk
    pos = np.asarray(segment_pos, dtype=np.int64).reshape(B, T)
    lens = (np.full(B, T, dtype=np.int64) if kv_valid_len is None
            else np.asarray(kv_valid_len, dtype=np.int64).reshape(B))
    q, k, v = project_qkv(x, w_q, w_kv, H, Hk, d_h)
    q_tilde = query_scale * rope(rms_norm(q, gamma_q), pos[:, :, None], rope_theta, rope_scale)
    k_rope = rope(rms_norm(k, gamma_k), pos[:, :, None], rope_theta, rope_scale)
    kc, vc = prefill_cache(x, pos, w_kv, gamma_k, k_cache, v_cache, num_kv_heads=Hk,
                           head_dim=d_h, rope_theta=rope_theta, rope_scale=rope_scale,
                           kv_valid_len=lens)
    o = np.empty((B, T, H, d_h), dtype=np.float64)
    t_idx = start + np.arange(T)
    s_idx = np.arange(start + T)
    for b in range(B):
        ok = allowed_mask(t_idx, s_idx, attn_type, window, start + lens[b])
        for kh in range(Hk):
            kb = np.concatenate([np.asarray(k_cache[b, :start, kh], dtype=np.float64),
                                 k_rope[b, :, kh]])
            vb = np.concatenate([np.asarray(v_cache[b, :start, kh], dtype=np.float64),
                                 v[b, :, kh]])
            o[b, :, kh * G:(kh + 1) * G] = attention_core(q_tilde[b, :, kh * G:(kh + 1) * G],
                                                          kb, vb, ok)
    y = o.reshape(B, T, H * d_h) @ np.asarray(w_o, dtype=np.float64).T
    return y, kc, vc


def gelu_tanh(u):
    """The tanh form of GELU (the Flax default the "Full Gemma 3 Block" page
    names for the MLP): 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (u + 0.044715 * u ** 3)))


def feed_forward(u, w_gating, w_linear):
    """GeGLU MLP ("Full Gemma 3 Block", How it works, MLP):
    FFN(u) = (GELU(u W_g) * (u W_u)) W_d. Layouts (readings): w_gating
    [2, D_ff, D] as stored with the transposed gating einsum (slice 0 = W_g,
    slice 1 = W_u, each contracted over D); w_linear [D, D_ff], output-major
    (W_d of shape (D_ff, D) transposed)."""
    u = np.asarray(u, dtype=np.float64)
    wg = np.asarray(w_gating, dtype=np.float64)
    gate = u @ wg[0].T
    up = u @ wg[1].T
    return (gelu_tanh(gate) * up) @ np.asarray(w_linear, dtype=np.float64).T


def block_prefill(x, segment_pos, attn_weights: dict, pre_attn_norm, post_attn_norm,
                  pre_ffw_norm, post_ffw_norm, w_gating, w_linear, *, num_heads: int,
                  num_kv_heads: int, head_dim: int, attn_type: str, window: int,
                  rope_theta: float, rope_scale: float, query_scale: float,
                  kv_valid_len=None):
    """One Gemma 3 block over the residual stream x [B,T,D] ("Full Gemma 3
    Block", How it works): a = post-norm(Attn(pre-norm(x))), h = x + a,
    m = post-norm(FFN(pre-norm(h))), y = h + m. Each norm is RMSNorm over D
    with (1 + gamma) and eps = 1e-6; Attn is `prefill` above."""
    x = np.asarray(x, dtype=np.float64)
    w = attn_weights
    a = prefill(rms_norm(x, pre_attn_norm), segment_pos, w["w_q"], w["w_kv"], w["w_o"],
                w["gamma_q"], w["gamma_k"], num_heads=num_heads, num_kv_heads=num_kv_heads,
                head_dim=head_dim, attn_type=attn_type, window=window, rope_theta=rope_theta,
                rope_scale=rope_scale, query_scale=query_scale, kv_valid_len=kv_valid_len)
    h = x + rms_norm(a, post_attn_norm)
    m = feed_forward(rms_norm(h, pre_ffw_norm), w_gating, w_linear)
    return h + rms_norm(m, post_ffw_norm)


def block_decode(x, segment_pos, attn_weights: dict, pre_attn_norm, post_attn_norm,
                 pre_ffw_norm, post_ffw_norm, w_gating, w_linear, k_cache, v_cache, *,
                 num_heads: int, num_kv_heads: int, head_dim: int, attn_type: str, window: int,
                 rope_theta: float, rope_scale: float, query_scale: float):
    """One decode step of a whole block ("Full Gemma 3 Block" around the
    decode step of "Gemma 3 Attention Block", Cache): the attention sublayer
    is `decode` on the pre-normed token (the cache holds keys and values of
    the pre-normed stream), the rest as in block_prefill. Returns y [B,1,D]
    and the (k, v) written at slot segment_pos[b]."""
    x = np.asarray(x, dtype=np.float64)
    w = attn_weights
    a, k_new, v_new = decode(rms_norm(x, pre_attn_norm), segment_pos, w["w_q"], w["w_kv"],
                             w["w_o"], w["gamma_q"], w["gamma_k"], k_cache, v_cache,
                             num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                             attn_type=attn_type, window=window, rope_theta=rope_theta,
                             rope_scale=rope_scale, query_scale=query_scale)
    h = x + rms_norm(a, post_attn_norm)
    m = feed_forward(rms_norm(h, pre_ffw_norm), w_gating, w_linear)
    return h + rms_norm(m, post_ffw_norm), k_new, v_new


def stack_prefill(x, segment_pos, layers: list, *, num_heads: int, num_kv_heads: int,
                  head_dim: int, window: int, local_rope=(1e4, 1.0), global_rope=(1e6, 8.0),
                  query_scale: float, kv_valid_len=None):
    """A stack of Gemma 3 blocks ("Global vs Local Layer Routing", How it
    works; "Full Gemma 3 Block"): layer l is a block of type
    layer_attn_type(l, len(layers)) with that type's (theta, scale) and, when
    local, the window; each layer's output is the next layer's input. layers:
    one dict per layer with the attention weights and the block weights
    (pre_attn_norm, post_attn_norm, pre_ffw_norm, post_ffw_norm, w_gating,
    w_linear)."""
    n = len(layers)
    h = np.asarray(x, dtype=np.float64)
    for l, w in enumerate(layers):
        t = layer_attn_type(l, n)
        theta, scale = local_rope if t == LOCAL_SLIDING else global_rope
        h = block_prefill(h, segment_pos, w, w["pre_attn_norm"], w["post_attn_norm"],
                          w["pre_ffw_norm"], w["post_ffw_norm"], w["w_gating"], w["w_linear"],
                          num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                          attn_type=t, window=window, rope_theta=theta, rope_scale=scale,
                          query_scale=query_scale, kv_valid_len=kv_valid_len)
    return h


def _layer_rope(l, n, local_rope, global_rope):
    t = layer_attn_type(l, n)
    theta, scale = local_rope if t == LOCAL_SLIDING else global_rope
    return t, theta, scale


def stack_prefill_cache(x, segment_pos, layers: list, k_caches: list, v_caches: list, *,
                        num_heads: int, num_kv_heads: int, head_dim: int, window: int,
                        local_rope=(1e4, 1.0), global_rope=(1e6, 8.0), query_scale: float,
                        kv_valid_len=None):
    """stack_prefill that also fills one left-aligned cache per layer ("Global
    vs Local Layer Routing", How it works: each layer attends with its own
    type; "Gemma 3 Attention Block", How it works, Cache). Layer l's cache
    receives the rotated keys and the values of that layer's own attention
    input, the pre-attention-normed stream, as prefill_cache writes them (with
    layer l's theta and scale). Returns y and the list of fp64 (k, v) caches."""
    n = len(layers)
    h = np.asarray(x, dtype=np.float64)
    caches = []
    for l, w in enumerate(layers):
        t, theta, scale = _layer_rope(l, n, local_rope, global_rope)
        caches.append(prefill_cache(rms_norm(h, w["pre_attn_norm"]), segment_pos, w["w_kv"],
                                    w["gamma_k"], k_caches[l], v_caches[l],
                                    num_kv_heads=num_kv_heads, head_dim=head_dim,
                                    rope_theta=theta, rope_scale=scale,
                                    kv_valid_len=kv_valid_len))
        h = block_prefill(h, segment_pos, w, w["pre_attn_norm"], w["post_attn_norm"],
                          w["pre_ffw_norm"], w["post_ffw_norm"], w["w_gating"], w["w_linear"],
                          num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                          attn_type=t, window=window, rope_theta=theta, rope_scale=scale,
                          query_scale=query_scale, kv_valid_len=kv_valid_len)
    return h, caches


def stack_decode(x, segment_pos, layers: list, k_caches: list, v_caches: list, *,
                 num_heads: int, num_kv_heads: int, head_dim: int, window: int,
                 local_rope=(1e4, 1.0), global_rope=(1e6, 8.0), query_scale: float):
    """One decode step of a routed stack: layer l is block_decode with the
    routed type, that type's (theta, scale) and, when local, the window,
    against layer l's own cache; each layer's output feeds the next. Returns
    y [B,1,D] and, per layer, the (k, v) written at slot segment_pos[b]."""
    n = len(layers)
    h = np.asarray(x, dtype=np.float64)
    written = []
    for l, w in enumerate(layers):
        t, theta, scale = _layer_rope(l, n, local_rope, global_rope)
        h, k_new, v_new = block_decode(
            h, segment_pos, w, w["pre_attn_norm"], w["post_attn_norm"], w["pre_ffw_norm"],
            w["post_ffw_norm"], w["w_gating"], w["w_linear"], k_caches[l], v_caches[l],
            num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim, attn_type=t,
            window=window, rope_theta=theta, rope_scale=scale, query_scale=query_scale)
        written.append((k_new, v_new))
    return h, written


def kv_cache_bytes(num_layers: int, batch: int, slots: int, num_kv_heads: int, head_dim: int,
                   window: int, elem_bytes: int, local_window_only: bool) -> int:
    """K and V cache bytes of a stack ("Gemma 3 Attention Block", Overview, and
    "Global vs Local Layer Routing": local layers only ever read their last W
    positions). Every layer holds K and V of [batch, S, H_kv, d_h]; with
    local_window_only a local layer holds min(W, S) slots instead."""
    per_slot = 2 * batch * num_kv_heads * head_dim * elem_bytes
    total = 0
    for l in range(num_layers):
        local = layer_attn_type(l, num_layers) == LOCAL_SLIDING
        total += per_slot * (min(window, slots) if local and local_window_only else slots)
    return total


def _prefill_rows(x, segment_pos, w_q, w_kv, w_o, gamma_q, gamma_k, rows, H, Hk, d_h,
                  attn_type, window, rope_theta, rope_scale, query_scale, kv_valid_len):
    """Selected query rows of prefill (same steps as the full computation)."""
    B, T, _ = x.shape
    G = H // Hk
    rows = np.unique(rows)
    if rows[0] < 0 or rows[-1] >= T:
        raise ValueError("query row out of range")
    lens = (np.full(B, T, dtype=np.int64) if kv_valid_len is None
            else np.asarray(kv_valid_len, dtype=np.int64).reshape(B))
    k_hi = int(rows[-1])
    k_lo = max(0, int(rows[0]) - window + 1) if attn_type == LOCAL_SLIDING else 0
    s_idx = np.arange(k_lo, k_hi + 1)
    pos = np.asarray(segment_pos, dtype=np.int64).reshape(B, T)
    w_q = np.asarray(w_q, dtype=np.float64)
    w_kv = np.asarray(w_kv, dtype=np.float64)
    n_k = Hk * d_h
    y = np.empty((B, len(rows), np.asarray(w_o).shape[0]), dtype=np.float64)
    for b in range(B):
        xq = np.asarray(x[b, rows], dtype=np.float64)
        xk = np.asarray(x[b, k_lo:k_hi + 1], dtype=np.float64)
        q = (xq @ w_q.T).reshape(len(rows), H, d_h)
        kv = xk @ w_kv.T
        k = kv[:, :n_k].reshape(-1, Hk, d_h)
        v = kv[:, n_k:].reshape(-1, Hk, d_h)
        q_t = query_scale * rope(rms_norm(q, gamma_q), pos[b, rows][:, None], rope_theta,
                                 rope_scale)
        k_r = rope(rms_norm(k, gamma_k), pos[b, k_lo:k_hi + 1][:, None], rope_theta,
                   rope_scale)
        ok = allowed_mask(rows, s_idx, attn_type, window, lens[b])
        o = np.empty((len(rows), H, d_h), dtype=np.float64)
        for kh in range(Hk):
            o[:, kh * G:(kh + 1) * G] = attention_core(q_t[:, kh * G:(kh + 1) * G],
                                                       k_r[:, kh], v[:, kh], ok)
        y[b] = o.reshape(len(rows), H * d_h) @ np.asarray(w_o, dtype=np.float64).T
    return y


# --------------------------------------------------------------------------
# Decode: one token against a left-aligned cache
# ("Gemma 3 Attention Block", How it works: Cache)
# --------------------------------------------------------------------------
def decode(x, segment_pos, w_q, w_kv, w_o, gamma_q, gamma_k, k_cache, v_cache, *,
           num_heads: int, num_kv_heads: int, head_dim: int,
           attn_type: str, window: int, rope_theta: float, rope_scale: float,
           query_scale: float, return_intermediates=False):
    """One decode step.

    x [B,1,D]; segment_pos [B,1] = query position t_b = the slot it writes;
    k_cache, v_cache [B,S,H_kv,d_h] hold rotated keys and values at slots
    0..t_b-1 (slot = position). The new token's rotated key and its value go
    to slot t_b; it then attends to slots s <= t_b (and s > t_b - W on local
    layers). Slots past t_b get zero weight under the mask, so only slots
    0..t_b are read. Returns y [B,1,D] and the (k, v) written at slot t_b.
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, _ = x.shape
    if T != 1:
        raise ValueError("decode takes one token per row")
    H, Hk, d_h = num_heads, num_kv_heads, head_dim
    G = H // Hk
    pos = np.asarray(segment_pos, dtype=np.int64).reshape(B)
    S = k_cache.shape[1]

    q, k, v = project_qkv(x, w_q, w_kv, H, Hk, d_h)
    q_hat = rms_norm(q, gamma_q)
    k_hat = rms_norm(k, gamma_k)
    q_rope = rope(q_hat, pos[:, None, None], rope_theta, rope_scale)
    k_rope = rope(k_hat, pos[:, None, None], rope_theta, rope_scale)
    q_tilde = query_scale * q_rope

    o = np.empty((B, 1, H, d_h), dtype=np.float64)
    for b in range(B):
        t = int(pos[b])
        if not 0 <= t < S:
            raise ValueError(f"position {t} outside the cache of length {S}")
        s_idx = np.arange(t + 1)
        ok = allowed_mask(np.array([t]), s_idx, attn_type, window, t + 1)
        for kh in range(Hk):
            kb = np.empty((t + 1, d_h), dtype=np.float64)
            vb = np.empty((t + 1, d_h), dtype=np.float64)
            kb[:t] = np.asarray(k_cache[b, :t, kh, :], dtype=np.float64)
            vb[:t] = np.asarray(v_cache[b, :t, kh, :], dtype=np.float64)
            kb[t] = k_rope[b, 0, kh]
            vb[t] = v[b, 0, kh]
            qb = q_tilde[b, :, kh * G:(kh + 1) * G, :]
            o[b, :, kh * G:(kh + 1) * G, :] = attention_core(qb, kb, vb, ok)

    y = o.reshape(B, 1, H * d_h) @ np.asarray(w_o, dtype=np.float64).T
    k_new, v_new = k_rope[:, 0], v[:, 0]
    if not return_intermediates:
        return y, k_new, v_new
    return y, k_new, v_new, dict(q=q, q_hat=q_hat, q_tilde=q_tilde, o=o)
