"""ctypes binding of libgemma3_attn.so (argument marshalling only).

Every step of the attention block runs in the library's HIP kernels; this
module checks tensor dtypes, devices and contiguity, allocates outputs and the
workspace with torch, and passes device pointers plus torch's current HIP
stream through the C ABI declared in include/gemma3_attn.h. There is no
fallback: if the library is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemma3_attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m global_layers_amd.build` "
        "(there is no CPU or PyTorch fallback)")

_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- C types
GLOBAL, LOCAL_SLIDING = 0, 1
F32, BF16 = 0, 1
OK = 0
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_WINDOW", 4: "ERR_DTYPE",
          5: "ERR_ROPE", 6: "ERR_WORKSPACE", 7: "ERR_UNSUPPORTED", 8: "ERR_HIP",
          9: "ERR_ALIGN", 10: "ERR_SCRATCH"}

STAGE_QKV_PROJ, STAGE_QK_NORM, STAGE_ATTN, STAGE_OUT_PROJ, STAGE_ALL = 1, 2, 4, 8, 15
STAGE_FORCE_EXACT_MAX = 16  # diagnostic: attention takes the exact-row-maximum pass
STAGE_FORCE_BOUND_REF = 32  # diagnostic: attention never takes the zero reference
DSTAGE_QKV_PROJ, DSTAGE_QK_NORM, DSTAGE_ATTN, DSTAGE_OUT_PROJ, DSTAGE_ALL = 1, 2, 4, 8, 15

_ATTN_TYPES = {"GLOBAL": GLOBAL, "LOCAL_SLIDING": LOCAL_SLIDING, GLOBAL: GLOBAL,
               LOCAL_SLIDING: LOCAL_SLIDING}
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
                ("H", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("attn_type", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rope_scale", ctypes.c_float),
                ("query_scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("w_q", ctypes.c_void_p), ("w_kv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("gamma_q", ctypes.c_void_p), ("gamma_k", ctypes.c_void_p)]


class WsLayout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_size_t), ("qkv", ctypes.c_size_t),
                ("q", ctypes.c_size_t), ("k", ctypes.c_size_t), ("vt", ctypes.c_size_t),
                ("o", ctypes.c_size_t), ("part", ctypes.c_size_t), ("ypart", ctypes.c_size_t),
                ("attn_part", ctypes.c_size_t), ("T_pad", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32), ("ksplit_qkv", ctypes.c_int32),
                ("ksplit_out", ctypes.c_int32)]


_P = ctypes.c_void_p
_lib.gemma3_attn_abi_version.restype = ctypes.c_int
_lib.gemma3_attn_status_string.restype = ctypes.c_char_p
_lib.gemma3_attn_status_string.argtypes = [ctypes.c_int]
_lib.gemma3_layer_attn_type.restype = ctypes.c_int
_lib.gemma3_layer_attn_type.argtypes = [ctypes.c_int32, ctypes.c_int32]
_lib.gemma3_attn_workspace_bytes.restype = ctypes.c_size_t
_lib.gemma3_attn_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32]
_lib.gemma3_attn_prefill_chunk_workspace_bytes.restype = ctypes.c_size_t
_lib.gemma3_attn_prefill_chunk_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32]
_lib.gemma3_attn_workspace_layout.restype = ctypes.c_int
_lib.gemma3_attn_workspace_layout.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                              ctypes.POINTER(WsLayout)]
class BlockWeights(ctypes.Structure):
    _fields_ = [("attn", Weights), ("pre_attn_norm", ctypes.c_void_p),
                ("post_attn_norm", ctypes.c_void_p), ("pre_ffw_norm", ctypes.c_void_p),
                ("post_ffw_norm", ctypes.c_void_p), ("w_gating", ctypes.c_void_p),
                ("w_linear", ctypes.c_void_p)]


_lib.gemma3_block_workspace_bytes.restype = ctypes.c_size_t
_lib.gemma3_block_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32]
_lib.gemma3_block_prefill.restype = ctypes.c_int
_lib.gemma3_block_prefill.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32, _P, _P, _P,
                                      ctypes.POINTER(BlockWeights), _P, _P, ctypes.c_size_t, _P]
class StackConfig(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("window", ctypes.c_int32),
                ("local_theta", ctypes.c_float), ("local_scale", ctypes.c_float),
                ("global_theta", ctypes.c_float), ("global_scale", ctypes.c_float)]


_lib.gemma3_stack_workspace_bytes.restype = ctypes.c_size_t
_lib.gemma3_stack_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                              ctypes.POINTER(StackConfig)]
_lib.gemma3_stack_prefill.restype = ctypes.c_int
_lib.gemma3_stack_prefill.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                      ctypes.POINTER(StackConfig), _P, _P, _P,
                                      ctypes.POINTER(BlockWeights), _P, _P, ctypes.c_size_t, _P]
_lib.gemma3_block_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.gemma3_block_decode_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                                     ctypes.c_int32]
_lib.gemma3_block_decode.restype = ctypes.c_int
_lib.gemma3_block_decode.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32, _P, _P,
                                     ctypes.POINTER(BlockWeights), _P, _P, ctypes.c_int32, _P,
                                     _P, ctypes.c_size_t, _P]
_PP = ctypes.POINTER(ctypes.c_void_p)
_lib.gemma3_stack_prefill_cache.restype = ctypes.c_int
_lib.gemma3_stack_prefill_cache.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                            ctypes.POINTER(StackConfig), _P, _P, _P,
                                            ctypes.POINTER(BlockWeights), _PP, _PP,
                                            ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]
_lib.gemma3_stack_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.gemma3_stack_decode_workspace_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                                     ctypes.POINTER(StackConfig), ctypes.c_int32]
_lib.gemma3_stack_decode.restype = ctypes.c_int
_lib.gemma3_stack_decode.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32,
                                     ctypes.POINTER(StackConfig), _P, _P,
                                     ctypes.POINTER(BlockWeights), _PP, _PP, ctypes.c_int32, _P,
                                     _P, ctypes.c_size_t, _P]
_lib.gemma3_kv_cache_bytes.restype = ctypes.c_size_t
_lib.gemma3_kv_cache_bytes.argtypes = [ctypes.c_int32] * 8


class KvFootprint(ctypes.Structure):
    _fields_ = [("n_local", ctypes.c_int32), ("n_global", ctypes.c_int32),
                ("local_bytes", ctypes.c_size_t), ("global_bytes", ctypes.c_size_t),
                ("local_window_bytes", ctypes.c_size_t)]


_lib.gemma3_attn_decode_static.restype = ctypes.c_int
_lib.gemma3_attn_decode_static.argtypes = [ctypes.POINTER(Desc), _P, _P, ctypes.POINTER(Weights),
                                           _P, _P, ctypes.c_int32, _P, _P]
STATIC_SCRATCH_BYTES = 64 << 20   # GEMMA3_STATIC_SCRATCH_BYTES
_lib.gemma3_kv_cache_footprint.restype = ctypes.c_int
_lib.gemma3_kv_cache_footprint.argtypes = [ctypes.c_int32] * 7 + [ctypes.POINTER(KvFootprint)]
_PREFILL_ARGS = [ctypes.POINTER(Desc), _P, _P, _P, ctypes.POINTER(Weights), _P, _P,
                 ctypes.c_size_t, _P]
_DECODE_ARGS = [ctypes.POINTER(Desc), _P, _P, ctypes.POINTER(Weights), _P, _P, ctypes.c_int32,
                _P, _P, ctypes.c_size_t, _P]
for name, args in (("gemma3_attn_prefill", _PREFILL_ARGS),
                   ("gemma3_attn_prefill_stages", _PREFILL_ARGS + [ctypes.c_uint32]),
                   ("gemma3_attn_prefill_cache",
                    [ctypes.POINTER(Desc), _P, _P, _P, ctypes.POINTER(Weights), _P, _P,
                     ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
                   ("gemma3_attn_prefill_chunk",
                    [ctypes.POINTER(Desc), _P, _P, _P, ctypes.POINTER(Weights), _P, _P,
                     ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
                   ("gemma3_attn_decode", _DECODE_ARGS),
                   ("gemma3_attn_decode_stages", _DECODE_ARGS + [ctypes.c_uint32])):
    fn = getattr(_lib, name)
    fn.restype = ctypes.c_int
    fn.argtypes = args

EXPORTED = ("gemma3_attn_workspace_bytes", "gemma3_attn_prefill", "gemma3_attn_decode",
            "gemma3_layer_attn_type", "gemma3_attn_status_string", "gemma3_attn_abi_version",
            "gemma3_attn_workspace_layout", "gemma3_attn_prefill_stages",
            "gemma3_attn_decode_stages", "gemma3_attn_prefill_cache",
            "gemma3_attn_prefill_chunk", "gemma3_attn_prefill_chunk_workspace_bytes",
            "gemma3_block_prefill", "gemma3_block_workspace_bytes", "gemma3_stack_prefill",
            "gemma3_stack_workspace_bytes", "gemma3_kv_cache_bytes", "gemma3_block_decode",
            "gemma3_block_decode_workspace_bytes", "gemma3_stack_prefill_cache",
            "gemma3_stack_decode", "gemma3_stack_decode_workspace_bytes",
            "gemma3_kv_cache_footprint", "gemma3_attn_decode_static")


class Gemma3AttnError(ValueError):
    def __init__(self, status: int):
        self.status = status
        msg = _lib.gemma3_attn_status_string(status).decode()
        super().__init__(f"{STATUS.get(status, status)}: {msg}")


def _check(status: int):
    if status != OK:
        raise Gemma3AttnError(status)


def abi_version() -> int:
    return _lib.gemma3_attn_abi_version()


def layer_attn_type(layer: int, num_layers: int) -> int:
    return _lib.gemma3_layer_attn_type(layer, num_layers)


def make_desc(*, B, T, D, H, H_kv, d_h, attn_type, window, rope_theta, rope_scale,
              query_scale, dtype) -> Desc:
    dt = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    at = _ATTN_TYPES.get(attn_type, attn_type)
    return Desc(int(B), int(T), int(D), int(H), int(H_kv), int(d_h), int(at), int(window),
                float(rope_theta), float(rope_scale), float(query_scale), dt)


def workspace_bytes(desc: Desc, S: int = 0) -> int:
    return _lib.gemma3_attn_workspace_bytes(ctypes.byref(desc), S)


def workspace_layout(desc: Desc, S: int = 0) -> WsLayout:
    L = WsLayout()
    _check(_lib.gemma3_attn_workspace_layout(ctypes.byref(desc), S, ctypes.byref(L)))
    return L


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(t, dtype, name, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _weights(w: dict, dtype, device) -> Weights:
    for k in ("w_q", "w_kv", "w_o", "gamma_q", "gamma_k"):
        _dev_tensor(w[k], dtype, k, device)
    return Weights(*(w[k].data_ptr() for k in ("w_q", "w_kv", "w_o", "gamma_q", "gamma_k")))


def fused_qkv_weights(w_qkv, w_o, gamma_q, gamma_k, *, H: int, d_h: int) -> dict:
    """Weights of a layer with H_kv == H whose projections are one fused matrix.

    "Gemma 3 Attention Block", How it works, projections: with as many KV
    heads as query heads a single qkv projection yields Q, K and V. w_qkv is
    [3*H*d_h, D], output-major, Q heads then K heads then V heads; w_q and
    w_kv become views into it (no copy): the library reads the Q rows and the
    K/V rows through two pointers that here point into one buffer.
    """
    n = H * d_h
    if w_qkv.dim() != 2 or w_qkv.shape[0] != 3 * n:
        raise ValueError("w_qkv must be [3 * H * d_h, D]")
    if not w_qkv.is_contiguous():
        raise ValueError("w_qkv must be contiguous")
    return dict(w_q=w_qkv[:n], w_kv=w_qkv[n:], w_o=w_o, gamma_q=gamma_q, gamma_k=gamma_k)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def new_workspace(desc: Desc, S: int = 0, device="cuda") -> torch.Tensor:
    n = workspace_bytes(desc, S)
    if n == 0:
        _check(_lib.gemma3_attn_workspace_layout(ctypes.byref(desc), S, ctypes.byref(WsLayout())))
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill(x, segment_pos, weights: dict, *, H, H_kv, d_h, attn_type, window, rope_theta,
            rope_scale, query_scale, kv_valid_len=None, workspace=None, y=None,
            stages: int = STAGE_ALL, k_cache=None, v_cache=None):
    """y [B,T,D] = attention layer over x [B,T,D] (see gemma3_attn_prefill).

    With k_cache and v_cache ([B,S,H_kv,d_h]) the call also writes every valid
    token's rotated key and value to slot segment_pos[b,t]
    (gemma3_attn_prefill_cache; all stages run)."""
    dev = x.device
    B, T, D = x.shape
    desc = make_desc(B=B, T=T, D=D, H=H, H_kv=H_kv, d_h=d_h, attn_type=attn_type,
                     window=window, rope_theta=rope_theta, rope_scale=rope_scale,
                     query_scale=query_scale, dtype=x.dtype)
    _dev_tensor(x, x.dtype, "x", dev)
    _dev_tensor(segment_pos, torch.int32, "segment_pos", dev)
    if segment_pos.shape != (B, T):
        raise ValueError("segment_pos must be [B, T]")
    if kv_valid_len is not None:
        _dev_tensor(kv_valid_len, torch.int32, "kv_valid_len", dev)
        if kv_valid_len.shape != (B,):
            raise ValueError("kv_valid_len must be [B]")
    w = _weights(weights, x.dtype, dev)
    if workspace is None:
        workspace = new_workspace(desc, 0, dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    if (k_cache is None) != (v_cache is None):
        raise ValueError("k_cache and v_cache go together")
    if k_cache is not None:
        if stages != STAGE_ALL:
            raise ValueError("a cache-filling prefill runs every stage")
        S = k_cache.shape[1]
        for n, c in (("k_cache", k_cache), ("v_cache", v_cache)):
            _dev_tensor(c, x.dtype, n, dev)
            if c.shape != (B, S, H_kv, d_h):
                raise ValueError(f"{n} must be [B, S, H_kv, d_h]")
        _check(_lib.gemma3_attn_prefill_cache(
            ctypes.byref(desc), _ptr(x), _ptr(segment_pos), _ptr(kv_valid_len), ctypes.byref(w),
            _ptr(k_cache), _ptr(v_cache), S, _ptr(y), _ptr(workspace), workspace.numel(),
            _stream()))
        return y
    _check(_lib.gemma3_attn_prefill_stages(
        ctypes.byref(desc), _ptr(x), _ptr(segment_pos), _ptr(kv_valid_len), ctypes.byref(w),
        _ptr(y), _ptr(workspace), workspace.numel(), _stream(), stages))
    return y


def prefill_chunk(x, segment_pos, weights: dict, k_cache, v_cache, start: int, *, H, H_kv, d_h,
                  attn_type, window, rope_theta, rope_scale, query_scale, kv_valid_len=None,
                  workspace=None, y=None):
    """y [B,T,D] for tokens start..start+T-1 of rows whose first `start` tokens
    are in the caches [B,S,H_kv,d_h]; writes the chunk's slots
    (see gemma3_attn_prefill_chunk)."""
    dev = x.device
    B, T, D = x.shape
    S = k_cache.shape[1]
    desc = make_desc(B=B, T=T, D=D, H=H, H_kv=H_kv, d_h=d_h, attn_type=attn_type,
                     window=window, rope_theta=rope_theta, rope_scale=rope_scale,
                     query_scale=query_scale, dtype=x.dtype)
    _dev_tensor(x, x.dtype, "x", dev)
    _dev_tensor(segment_pos, torch.int32, "segment_pos", dev)
    if segment_pos.shape != (B, T):
        raise ValueError("segment_pos must be [B, T]")
    if kv_valid_len is not None:
        _dev_tensor(kv_valid_len, torch.int32, "kv_valid_len", dev)
        if kv_valid_len.shape != (B,):
            raise ValueError("kv_valid_len must be [B]")
    for n, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(c, x.dtype, n, dev)
        if c.shape != (B, S, H_kv, d_h):
            raise ValueError(f"{n} must be [B, S, H_kv, d_h]")
    w = _weights(weights, x.dtype, dev)
    if workspace is None:
        n = _lib.gemma3_attn_prefill_chunk_workspace_bytes(ctypes.byref(desc), start)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    _check(_lib.gemma3_attn_prefill_chunk(
        ctypes.byref(desc), _ptr(x), _ptr(segment_pos), _ptr(kv_valid_len), ctypes.byref(w),
        _ptr(k_cache), _ptr(v_cache), S, start, _ptr(y), _ptr(workspace), workspace.numel(),
        _stream()))
    return y


BLOCK_KEYS = ("pre_attn_norm", "post_attn_norm", "pre_ffw_norm", "post_ffw_norm", "w_gating",
              "w_linear")


def block_prefill(x, segment_pos, weights: dict, *, H, H_kv, d_h, attn_type, window, rope_theta,
                  rope_scale, query_scale, kv_valid_len=None, workspace=None, y=None):
    """y [B,T,D] = one Gemma 3 block over the residual stream x (see
    gemma3_block_prefill). weights: the attention's five tensors plus
    BLOCK_KEYS (norms [D], w_gating [2, D_ff, D], w_linear [D, D_ff])."""
    dev = x.device
    B, T, D = x.shape
    D_ff = weights["w_gating"].shape[1]
    desc = make_desc(B=B, T=T, D=D, H=H, H_kv=H_kv, d_h=d_h, attn_type=attn_type,
                     window=window, rope_theta=rope_theta, rope_scale=rope_scale,
                     query_scale=query_scale, dtype=x.dtype)
    _dev_tensor(x, x.dtype, "x", dev)
    _dev_tensor(segment_pos, torch.int32, "segment_pos", dev)
    if segment_pos.shape != (B, T):
        raise ValueError("segment_pos must be [B, T]")
    if kv_valid_len is not None:
        _dev_tensor(kv_valid_len, torch.int32, "kv_valid_len", dev)
        if kv_valid_len.shape != (B,):
            raise ValueError("kv_valid_len must be [B]")
    for k in BLOCK_KEYS:
        _dev_tensor(weights[k], x.dtype, k, dev)
    if weights["w_gating"].shape != (2, D_ff, D) or weights["w_linear"].shape != (D, D_ff):
        raise ValueError("w_gating must be [2, D_ff, D] and w_linear [D, D_ff]")
    bw = BlockWeights(_weights(weights, x.dtype, dev),
                      *(weights[k].data_ptr() for k in BLOCK_KEYS))
    if workspace is None:
        n = _lib.gemma3_block_workspace_bytes(ctypes.byref(desc), D_ff)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    _check(_lib.gemma3_block_prefill(ctypes.byref(desc), D_ff, _ptr(x), _ptr(segment_pos),
                                     _ptr(kv_valid_len), ctypes.byref(bw), _ptr(y),
                                     _ptr(workspace), workspace.numel(), _stream()))
    return y


def _stack_args(x, layers, H, H_kv, d_h, window, query_scale, local_rope, global_rope):
    dev = x.device
    B, T, D = x.shape
    n = len(layers)
    D_ff = layers[0]["w_gating"].shape[1]
    desc = make_desc(B=B, T=T, D=D, H=H, H_kv=H_kv, d_h=d_h, attn_type="GLOBAL", window=window,
                     rope_theta=global_rope[0], rope_scale=global_rope[1],
                     query_scale=query_scale, dtype=x.dtype)
    cfg = StackConfig(n, window, local_rope[0], local_rope[1], global_rope[0], global_rope[1])
    _dev_tensor(x, x.dtype, "x", dev)
    arr = (BlockWeights * n)()
    for l, w in enumerate(layers):
        for k in BLOCK_KEYS:
            _dev_tensor(w[k], x.dtype, k, dev)
        if w["w_gating"].shape != (2, D_ff, D) or w["w_linear"].shape != (D, D_ff):
            raise ValueError("every layer needs w_gating [2, D_ff, D] and w_linear [D, D_ff]")
        arr[l] = BlockWeights(_weights(w, x.dtype, dev), *(w[k].data_ptr() for k in BLOCK_KEYS))
    return desc, cfg, arr, D_ff


def _cache_arrays(k_caches, v_caches, n, B, H_kv, d_h, dtype, dev):
    """Host arrays of the per-layer cache device pointers (all [B, S, H_kv, d_h])."""
    if len(k_caches) != n or len(v_caches) != n:
        raise ValueError("one k and one v cache per layer")
    S = k_caches[0].shape[1]
    ka, va = (ctypes.c_void_p * n)(), (ctypes.c_void_p * n)()
    for l in range(n):
        for nm, c in (("k_cache", k_caches[l]), ("v_cache", v_caches[l])):
            _dev_tensor(c, dtype, nm, dev)
            if c.shape != (B, S, H_kv, d_h):
                raise ValueError(f"{nm} of layer {l} must be [B, S, H_kv, d_h]")
        ka[l], va[l] = k_caches[l].data_ptr(), v_caches[l].data_ptr()
    return ka, va, S


def stack_prefill(x, segment_pos, layers: list, *, H, H_kv, d_h, window, query_scale,
                  local_rope=(1e4, 1.0), global_rope=(1e6, 8.0), kv_valid_len=None,
                  workspace=None, y=None, k_caches=None, v_caches=None):
    """y [B,T,D] of a routed stack of blocks, one weights dict per layer (as
    block_prefill takes); layer l's type is layer_attn_type(l, len(layers))
    (see gemma3_stack_prefill). With k_caches / v_caches (one [B,S,H_kv,d_h]
    tensor per layer) every layer also fills its own cache
    (gemma3_stack_prefill_cache)."""
    dev = x.device
    B, T, D = x.shape
    desc, cfg, arr, D_ff = _stack_args(x, layers, H, H_kv, d_h, window, query_scale, local_rope,
                                       global_rope)
    _dev_tensor(segment_pos, torch.int32, "segment_pos", dev)
    if segment_pos.shape != (B, T):
        raise ValueError("segment_pos must be [B, T]")
    if kv_valid_len is not None:
        _dev_tensor(kv_valid_len, torch.int32, "kv_valid_len", dev)
    if workspace is None:
        nb = _lib.gemma3_stack_workspace_bytes(ctypes.byref(desc), D_ff, ctypes.byref(cfg))
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    if (k_caches is None) != (v_caches is None):
        raise ValueError("k_caches and v_caches go together")
    if k_caches is None:
        _check(_lib.gemma3_stack_prefill(ctypes.byref(desc), D_ff, ctypes.byref(cfg), _ptr(x),
                                         _ptr(segment_pos), _ptr(kv_valid_len), arr, _ptr(y),
                                         _ptr(workspace), workspace.numel(), _stream()))
        return y
    ka, va, S = _cache_arrays(k_caches, v_caches, len(layers), B, H_kv, d_h, x.dtype, dev)
    _check(_lib.gemma3_stack_prefill_cache(ctypes.byref(desc), D_ff, ctypes.byref(cfg), _ptr(x),
                                           _ptr(segment_pos), _ptr(kv_valid_len), arr, ka, va,
                                           S, _ptr(y), _ptr(workspace), workspace.numel(),
                                           _stream()))
    return y


def stack_decode(x, segment_pos, layers: list, k_caches, v_caches, *, H, H_kv, d_h, window,
                 query_scale, local_rope=(1e4, 1.0), global_rope=(1e6, 8.0), workspace=None,
                 y=None):
    """y [B,1,D]: one decode step of a routed stack, layer l against its own
    caches k_caches[l] / v_caches[l] (see gemma3_stack_decode)."""
    dev = x.device
    B, T, D = x.shape
    desc, cfg, arr, D_ff = _stack_args(x, layers, H, H_kv, d_h, window, query_scale, local_rope,
                                       global_rope)
    _dev_tensor(segment_pos, torch.int32, "segment_pos", dev)
    if segment_pos.numel() != B:
        raise ValueError("segment_pos must hold one position per row")
    ka, va, S = _cache_arrays(k_caches, v_caches, len(layers), B, H_kv, d_h, x.dtype, dev)
    if workspace is None:
        nb = _lib.gemma3_stack_decode_workspace_bytes(ctypes.byref(desc), D_ff,
                                                      ctypes.byref(cfg), S)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    _check(_lib.gemma3_stack_decode(ctypes.byref(desc), D_ff, ctypes.byref(cfg), _ptr(x),
                                    _ptr(segment_pos), arr, ka, va, S, _ptr(y), _ptr(workspace),
                                    workspace.numel(), _stream()))
    return y


def block_decode(x, segment_pos, weights: dict, k_cache, v_cache, *, H, H_kv, d_h, attn_type,
                 window, rope_theta, rope_scale, query_scale, workspace=None, y=None):
    """y [B,1,D]: one decode step of a whole block (see gemma3_block_decode);
    the caches hold this layer's pre-normed keys and values."""
    dev = x.device
    B, T, D = x.shape
    S = k_cache.shape[1]
    D_ff = weights["w_gating"].shape[1]
    desc = make_desc(B=B, T=T, D=D, H=H, H_kv=H_kv, d_h=d_h, attn_type=attn_type,
                     window=window, rope_theta=rope_theta, rope_scale=rope_scale,
                     query_scale=query_scale, dtype=x.dtype)
    _dev_tensor(x, x.dtype, "x", dev)
    _dev_tensor(segment_pos, torch.int32, "segment_pos", dev)
    if segment_pos.numel() != B:
        raise ValueError("segment_pos must hold one position per row")
    for n, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(c, x.dtype, n, dev)
        if c.shape != (B, S, H_kv, d_h):
            raise ValueError(f"{n} must be [B, S, H_kv, d_h]")
    for k in BLOCK_KEYS:
        _dev_tensor(weights[k], x.dtype, k, dev)
    if weights["w_gating"].shape != (2, D_ff, D) or weights["w_linear"].shape != (D, D_ff):
        raise ValueError("w_gating must be [2, D_ff, D] and w_linear [D, D_ff]")
    bw = BlockWeights(_weights(weights, x.dtype, dev),
                      *(weights[k].data_ptr() for k in BLOCK_KEYS))
    if workspace is None:
        n = _lib.gemma3_block_decode_workspace_bytes(ctypes.byref(desc), D_ff, S)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    _check(_lib.gemma3_block_decode(ctypes.byref(desc), D_ff, _ptr(x), _ptr(segment_pos),
                                    ctypes.byref(bw), _ptr(k_cache), _ptr(v_cache), S, _ptr(y),
                                    _ptr(workspace), workspace.numel(), _stream()))
    return y


def kv_cache_bytes(num_layers, B, S, H_kv, d_h, window, dtype, local_window_only) -> int:
    """K and V cache bytes of a stack (see gemma3_kv_cache_bytes)."""
    dt = _DTYPES.get(dtype, dtype)
    return _lib.gemma3_kv_cache_bytes(num_layers, B, S, H_kv, d_h, window, dt,
                                      1 if local_window_only else 0)


def kv_cache_footprint(num_layers, B, S, H_kv, d_h, window, dtype) -> dict:
    """Per-type K/V cache bytes of a routed stack (see gemma3_kv_cache_footprint)."""
    dt = _DTYPES.get(dtype, dtype)
    f = KvFootprint()
    _check(_lib.gemma3_kv_cache_footprint(num_layers, B, S, H_kv, d_h, window, dt,
                                          ctypes.byref(f)))
    return {k: getattr(f, k) for k, _ in KvFootprint._fields_}


def decode(x, segment_pos, weights: dict, k_cache, v_cache, *, H, H_kv, d_h, attn_type, window,
           rope_theta, rope_scale, query_scale, workspace=None, y=None,
           stages: int = DSTAGE_ALL):
    """y [B,1,D] for one token per row; writes slot segment_pos[b] of the caches."""
    dev = x.device
    B, T, D = x.shape
    S = k_cache.shape[1]
    desc = make_desc(B=B, T=T, D=D, H=H, H_kv=H_kv, d_h=d_h, attn_type=attn_type,
                     window=window, rope_theta=rope_theta, rope_scale=rope_scale,
                     query_scale=query_scale, dtype=x.dtype)
    _dev_tensor(x, x.dtype, "x", dev)
    _dev_tensor(segment_pos, torch.int32, "segment_pos", dev)
    if segment_pos.numel() != B:
        raise ValueError("segment_pos must hold one position per row")
    for n, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(c, x.dtype, n, dev)
        if c.shape != (B, S, H_kv, d_h):
            raise ValueError(f"{n} must be [B, S, H_kv, d_h]")
    w = _weights(weights, x.dtype, dev)
    if workspace is None:
        workspace = new_workspace(desc, S, dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    _check(_lib.gemma3_attn_decode_stages(
        ctypes.byref(desc), _ptr(x), _ptr(segment_pos), ctypes.byref(w), _ptr(k_cache),
        _ptr(v_cache), S, _ptr(y), _ptr(workspace), workspace.numel(), _stream(), stages))
    return y


def decode_static(x, segment_pos, weights: dict, k_cache, v_cache, *, H, H_kv, d_h, attn_type,
                  window, rope_theta, rope_scale, query_scale, y=None):
    """decode() without a workspace: the library's static per-GPU scratch
    (gemma3_attn_decode_static; nothing is allocated but y when not given)."""
    dev = x.device
    B, T, D = x.shape
    S = k_cache.shape[1]
    desc = make_desc(B=B, T=T, D=D, H=H, H_kv=H_kv, d_h=d_h, attn_type=attn_type,
                     window=window, rope_theta=rope_theta, rope_scale=rope_scale,
                     query_scale=query_scale, dtype=x.dtype)
    _dev_tensor(x, x.dtype, "x", dev)
    _dev_tensor(segment_pos, torch.int32, "segment_pos", dev)
    if segment_pos.numel() != B:
        raise ValueError("segment_pos must hold one position per row")
    for n, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(c, x.dtype, n, dev)
        if c.shape != (B, S, H_kv, d_h):
            raise ValueError(f"{n} must be [B, S, H_kv, d_h]")
    w = _weights(weights, x.dtype, dev)
    if y is None:
        y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    _check(_lib.gemma3_attn_decode_static(
        ctypes.byref(desc), _ptr(x), _ptr(segment_pos), ctypes.byref(w), _ptr(k_cache),
        _ptr(v_cache), S, _ptr(y), _stream()))
    return y


def prefill_intermediates(workspace: torch.Tensor, desc: Desc) -> dict:
    """Views of the prefill intermediates inside a workspace (see gemma3_ws_layout)."""
    L = workspace_layout(desc, 0)
    dt = torch.bfloat16 if desc.dtype == BF16 else torch.float32
    esz = 2 if desc.dtype == BF16 else 4
    B, T, H, Hk, d = desc.B, desc.T, desc.H, desc.H_kv, desc.d_h

    def view(off, shape):
        n = 1
        for s in shape:
            n *= s
        return workspace[off:off + n * esz].view(dt).view(shape)

    return dict(
        qkv=view(L.qkv, (B * T, (H + 2 * Hk) * d)),
        o=view(L.o, (B, T, H, d)),
        q=view(L.q, (B, H, T, d)),
        k=view(L.k, (B, Hk, L.T_pad, d)),
        vt=view(L.vt, (B, Hk, d, L.T_pad)),
        T_pad=L.T_pad)


def decode_intermediates(workspace: torch.Tensor, desc: Desc, S: int) -> dict:
    L = workspace_layout(desc, S)
    dt = torch.bfloat16 if desc.dtype == BF16 else torch.float32
    esz = 2 if desc.dtype == BF16 else 4
    B, H, d = desc.B, desc.H, desc.d_h
    q = workspace[L.q:L.q + B * H * d * 4].view(torch.float32).view(B, H, d)
    o = workspace[L.o:L.o + B * H * d * esz].view(dt).view(B, H, d)
    return dict(q=q, o=o, chunk=L.chunk, n_chunks=L.n_chunks)
