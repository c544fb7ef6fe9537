"""C-ABI checks that need no GPU: the library loads, exports every function
the public headers declare, and host validation returns each status before
anything is enqueued (fake device addresses are never dereferenced on these
paths)."""

import ctypes
import os
import re

import pytest

from global_layers_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in ("gemma3_attn.h", "gemma3_attn_stages.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(gemma3_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"gemma3_attn_prefill", "gemma3_attn_decode", "gemma3_attn_workspace_bytes",
            "gemma3_layer_attn_type", "gemma3_attn_status_string"} <= names
    so = ctypes.CDLL(lib.LIB_PATH)
    for n in sorted(names):
        assert hasattr(so, n), f"{n} declared but not exported"
    assert set(lib.EXPORTED) == names


def test_stage_constants_match_the_header():
    """Every GEMMA3_STAGE_* / GEMMA3_DSTAGE_* bit of the stages header has the
    same value in the Python binding (STAGE_* / DSTAGE_*)."""
    text = open(os.path.join(ROOT, "include", "gemma3_attn_stages.h")).read()
    defs = re.findall(r"#define GEMMA3_(D?STAGE_\w+)\s+(0x[0-9A-Fa-f]+)u", text)
    assert len(defs) >= 12
    for name, val in defs:
        assert getattr(lib, name) == int(val, 16), name


def test_abi_version_and_status_strings():
    assert lib.abi_version() == 3
    for st in range(10):
        assert lib._lib.gemma3_attn_status_string(st)
    assert lib._lib.gemma3_attn_status_string(99) == b"unknown status"


def test_layer_routing_helper():
    for n in (1, 5, 6, 7, 26, 34, 48, 62):
        types = [lib.layer_attn_type(l, n) for l in range(n)]
        assert types[0] == lib.LOCAL_SLIDING
        assert all((t == lib.GLOBAL) == (l % 6 == 5) for l, t in enumerate(types))
        assert types.count(lib.GLOBAL) == n // 6
    assert lib.layer_attn_type(-1, 6) == -1 and lib.layer_attn_type(6, 6) == -1


def _desc(**kw):
    d = dict(B=1, T=128, D=256, H=4, H_kv=1, d_h=64, attn_type="LOCAL_SLIDING", window=32,
             rope_theta=1e4, rope_scale=1.0, query_scale=0.125, dtype=lib.BF16)
    d.update(kw)
    return lib.make_desc(**d)


FAKE = 1 << 40  # 16-byte aligned address never touched by the validation paths


def _call_prefill(desc, ws_bytes=None, x=FAKE, pos=FAKE, y=FAKE, ws=FAKE, weights=None):
    w = weights or lib.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    n = lib.workspace_bytes(desc) if ws_bytes is None else ws_bytes
    return lib._lib.gemma3_attn_prefill(ctypes.byref(desc), x, pos, None, ctypes.byref(w), y, ws,
                                        n, None)


def _call_decode(desc, S=1024, ws_bytes=None, kc=FAKE, vc=FAKE):
    w = lib.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    n = lib.workspace_bytes(desc, S) if ws_bytes is None else ws_bytes
    return lib._lib.gemma3_attn_decode(ctypes.byref(desc), FAKE, FAKE, ctypes.byref(w), kc, vc,
                                       S, FAKE, FAKE, n, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(T=-1), 2), (dict(D=0), 2), (dict(H=0), 2), (dict(H_kv=0), 2),
    (dict(H=6, H_kv=4), 2), (dict(d_h=63), 2),
    (dict(attn_type=7), 4), (dict(dtype=5), 4),
    (dict(window=0), 3), (dict(window=-3), 3),
    (dict(rope_theta=0.0), 5), (dict(rope_scale=-1.0), 5), (dict(rope_theta=float("inf")), 5),
    (dict(query_scale=float("nan")), 5),
    (dict(d_h=96), 7), (dict(D=100), 7), (dict(d_h=512), 7),
    (dict(d_h=300, dtype=lib.F32), 7), (dict(d_h=48, dtype=lib.F32), 7),
    (dict(d_h=8, dtype=lib.F32), 7),
])
def test_prefill_validation_status(kw, status):
    assert _call_prefill(_desc(**kw), ws_bytes=1 << 40) == status
    if status != 7:
        assert lib.workspace_bytes(_desc(**kw)) == 0


def test_prefill_pointer_workspace_alignment_errors():
    d = _desc()
    assert lib._lib.gemma3_attn_prefill(None, FAKE, FAKE, None, None, FAKE, FAKE, 1, None) == 1
    assert _call_prefill(d, x=None) == 1
    assert _call_prefill(d, pos=None) == 1
    assert _call_prefill(d, y=None) == 1
    assert _call_prefill(d, weights=lib.Weights(FAKE, None, FAKE, FAKE, FAKE)) == 1
    assert _call_prefill(d, ws=None) == 6
    assert _call_prefill(d, ws_bytes=lib.workspace_bytes(d) - 1) == 6
    assert _call_prefill(d, x=FAKE + 2) == 9
    assert _call_prefill(d, ws=FAKE + 8) == 9
    assert _call_prefill(d, weights=lib.Weights(FAKE, FAKE + 4, FAKE, FAKE, FAKE)) == 9


def test_global_layer_ignores_window():
    d = _desc(attn_type="GLOBAL", window=0)
    assert lib.workspace_bytes(d) > 0


def test_decode_validation_status():
    d = _desc(T=1, d_h=128, H=4, H_kv=2, D=256)
    assert _call_decode(d, S=0) == 2
    assert _call_decode(_desc(T=2, d_h=128), S=16) == 2
    assert _call_decode(d, ws_bytes=16) == 6
    assert _call_decode(d, kc=None) == 1
    assert _call_decode(d, vc=FAKE + 2) == 9
    assert _call_decode(_desc(T=1, d_h=32, dtype=lib.F32, D=64), S=8, ws_bytes=1 << 30) == 7


def _call_prefill_cache(desc, S=512, kc=FAKE, vc=FAKE, x=FAKE, ws_bytes=None):
    w = lib.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    n = lib.workspace_bytes(desc) if ws_bytes is None else ws_bytes
    return lib._lib.gemma3_attn_prefill_cache(ctypes.byref(desc), x, FAKE, None,
                                              ctypes.byref(w), kc, vc, S, FAKE, FAKE, n, None)


def test_prefill_cache_validation_status():
    d = _desc()
    assert lib._lib.gemma3_attn_prefill_cache(None, FAKE, FAKE, None, None, FAKE, FAKE, 8,
                                              FAKE, FAKE, 1, None) == 1
    assert _call_prefill_cache(d, S=0) == 2
    assert _call_prefill_cache(_desc(B=0)) == 2
    assert _call_prefill_cache(d, kc=None) == 1
    assert _call_prefill_cache(d, vc=None) == 1
    assert _call_prefill_cache(d, kc=FAKE + 2) == 9
    assert _call_prefill_cache(d, x=None) == 1      # the prefill's own checks
    assert _call_prefill_cache(d, ws_bytes=16) == 6
    assert _call_prefill_cache(_desc(d_h=96), ws_bytes=1 << 40) == 7


def _call_prefill_chunk(desc, S=512, start=100, kc=FAKE, ws_bytes=None):
    w = lib.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    n = (lib._lib.gemma3_attn_prefill_chunk_workspace_bytes(ctypes.byref(desc), start)
         if ws_bytes is None else ws_bytes)
    return lib._lib.gemma3_attn_prefill_chunk(ctypes.byref(desc), FAKE, FAKE, None,
                                              ctypes.byref(w), kc, FAKE, S, start, FAKE, FAKE, n,
                                              None)


def test_prefill_chunk_validation_status():
    d = _desc()  # T = 128
    ws = lib._lib.gemma3_attn_prefill_chunk_workspace_bytes
    # the prefill's workspace plus room for split-KV partials; the attention
    # reads the cached keys in place, so the size does not grow with start
    assert ws(ctypes.byref(d), 0) > lib.workspace_bytes(d)
    assert ws(ctypes.byref(d), 1000) == ws(ctypes.byref(d), 0)
    assert ws(ctypes.byref(d), 1 << 30) == ws(ctypes.byref(d), 0)
    assert ws(ctypes.byref(d), -1) == 0
    assert _call_prefill_chunk(d, start=-1) == 2
    assert _call_prefill_chunk(d, S=227, start=100) == 2    # start + T > S
    assert _call_prefill_chunk(d, S=0, start=0) == 2
    assert _call_prefill_chunk(d, kc=None) == 1
    assert _call_prefill_chunk(d, kc=FAKE + 4) == 9
    assert _call_prefill_chunk(d, ws_bytes=lib.workspace_bytes(d)) == 6
    assert _call_prefill_chunk(_desc(d_h=96), ws_bytes=1 << 40) == 7


def test_block_validation_status():
    d = _desc()  # bf16, D = 256
    f = lib._lib.gemma3_block_workspace_bytes
    assert f(ctypes.byref(d), 512) > lib.workspace_bytes(d)
    assert f(ctypes.byref(d), 0) == 0
    assert f(ctypes.byref(d), 100) == 0                      # bf16 needs D_ff % 64 == 0
    assert f(ctypes.byref(_desc(dtype=lib.F32)), 100) > 0
    aw = lib.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)

    def call(D_ff=512, x=FAKE, y=FAKE + 4096, bw=None, n=None):
        bw = bw or lib.BlockWeights(aw, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
        n = f(ctypes.byref(d), D_ff) if n is None else n
        return lib._lib.gemma3_block_prefill(ctypes.byref(d), D_ff, x, FAKE, None,
                                             ctypes.byref(bw), y, FAKE, n, None)
    assert call(D_ff=0, n=1 << 40) == 2
    assert call(D_ff=96, n=1 << 40) == 7
    assert call(x=None) == 1
    assert call(bw=lib.BlockWeights(aw, FAKE, None, FAKE, FAKE, FAKE, FAKE)) == 1
    assert call(bw=lib.BlockWeights(aw, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE)) == 9
    assert call(y=FAKE) == 2                                   # y may not alias x
    assert call(n=16) == 6


def test_kv_cache_footprint_matches_oracle():
    import oracle as O
    for args in ((26, 1, 131072, 1, 256, 512), (34, 16, 131072, 8, 256, 1024),
                 (62, 2, 32768, 16, 128, 1024), (5, 1, 100, 1, 256, 512), (1, 3, 10, 2, 64, 4)):
        for dt, esz in ((lib.BF16, 2), (lib.F32, 4)):
            for only in (False, True):
                assert lib.kv_cache_bytes(*args, dt, only) == O.kv_cache_bytes(*args, esz, only)
    assert lib.kv_cache_bytes(0, 1, 10, 1, 64, 4, lib.BF16, True) == 0


def test_kv_cache_footprint_splits_by_routed_type():
    # local and global bytes each against the oracle's routing and its
    # whole-stack formula (a stack of only its local, or only its global, layers)
    import oracle as O
    for args in ((26, 1, 131072, 1, 256, 512), (62, 2, 32768, 16, 128, 1024), (7, 1, 100, 1, 64, 4)):
        n, B, S, Hk, d_h, Wn = args
        f = lib.kv_cache_footprint(*args, lib.BF16)
        types = O.layer_attn_types(n)
        assert (f["n_local"], f["n_global"]) == (types.count(O.LOCAL_SLIDING), types.count(O.GLOBAL))
        per_layer = O.kv_cache_bytes(1, B, S, Hk, d_h, Wn, 2, False)
        per_local_window = O.kv_cache_bytes(1, B, S, Hk, d_h, Wn, 2, True)
        assert f["global_bytes"] == f["n_global"] * per_layer
        assert f["local_bytes"] == f["n_local"] * per_layer
        assert f["local_window_bytes"] == f["n_local"] * per_local_window
        assert f["local_bytes"] + f["global_bytes"] == O.kv_cache_bytes(*args, 2, False)
        assert f["local_window_bytes"] + f["global_bytes"] == O.kv_cache_bytes(*args, 2, True)
    bad = lib.KvFootprint()
    assert lib._lib.gemma3_kv_cache_footprint(0, 1, 10, 1, 64, 4, lib.BF16, ctypes.byref(bad)) == 2
    assert lib._lib.gemma3_kv_cache_footprint(6, 1, 10, 1, 64, 0, lib.BF16, ctypes.byref(bad)) == 3
    assert lib._lib.gemma3_kv_cache_footprint(6, 1, 10, 1, 64, 4, 7, ctypes.byref(bad)) == 4
    assert lib._lib.gemma3_kv_cache_footprint(6, 1, 10, 1, 64, 4, lib.BF16, None) == 1


def test_stack_cache_and_decode_validation_status():
    d = _desc()
    cfg = lib.StackConfig(7, 64, 1e4, 1.0, 1e6, 8.0)
    aw = lib.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    good = lib.BlockWeights(aw, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    arr = (lib.BlockWeights * 7)(*([good] * 7))
    n = lib._lib.gemma3_stack_workspace_bytes(ctypes.byref(d), 512, ctypes.byref(cfg))
    caches = (ctypes.c_void_p * 7)(*([FAKE] * 7))
    holed = (ctypes.c_void_p * 7)(*([FAKE] * 6 + [None]))
    skew = (ctypes.c_void_p * 7)(*([FAKE] * 6 + [FAKE + 8]))
    pf = lambda kc, vc, S=64, ws=n: lib._lib.gemma3_stack_prefill_cache(  # noqa: E731
        ctypes.byref(d), 512, ctypes.byref(cfg), FAKE, FAKE, None, arr, kc, vc, S, FAKE + 4096,
        FAKE, ws, None)
    assert pf(None, caches) == 1
    assert pf(caches, holed) == 1
    assert pf(caches, skew) == 9
    assert pf(caches, caches, S=0) == 2
    assert pf(caches, caches, ws=16) == 6
    dd = _desc(T=1)
    nd = lib._lib.gemma3_stack_decode_workspace_bytes(ctypes.byref(dd), 512, ctypes.byref(cfg), 64)
    assert nd > 0
    assert lib._lib.gemma3_stack_decode_workspace_bytes(ctypes.byref(dd), 512, ctypes.byref(cfg),
                                                        0) == 0
    dc = lambda kc, vc, S=64, ws=nd, desc=dd: lib._lib.gemma3_stack_decode(  # noqa: E731
        ctypes.byref(desc), 512, ctypes.byref(cfg), FAKE, FAKE, arr, kc, vc, S, FAKE + 4096,
        FAKE, ws, None)
    assert dc(caches, holed) == 1
    assert dc(caches, skew) == 9
    assert dc(caches, caches, S=0) == 2
    assert dc(caches, caches, ws=16) == 6
    assert dc(caches, caches, desc=d) == 2                  # T != 1


def test_stack_validation_status():
    d = _desc()
    cfg = lib.StackConfig(7, 64, 1e4, 1.0, 1e6, 8.0)
    f = lib._lib.gemma3_stack_workspace_bytes
    n = f(ctypes.byref(d), 512, ctypes.byref(cfg))
    assert n > lib._lib.gemma3_block_workspace_bytes(ctypes.byref(d), 512)
    assert f(ctypes.byref(d), 512, ctypes.byref(lib.StackConfig(0, 64, 1e4, 1.0, 1e6, 8.0))) == 0
    assert f(ctypes.byref(d), 512, ctypes.byref(lib.StackConfig(6, 0, 1e4, 1.0, 1e6, 8.0))) == 0
    aw = lib.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    good = lib.BlockWeights(aw, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    arr = (lib.BlockWeights * 7)(*([good] * 7))
    call = lambda a, ws=n: lib._lib.gemma3_stack_prefill(  # noqa: E731
        ctypes.byref(d), 512, ctypes.byref(cfg), FAKE, FAKE, None, a, FAKE + 4096, FAKE, ws, None)
    bad = (lib.BlockWeights * 7)(*([good] * 6 + [lib.BlockWeights(aw, FAKE, FAKE, FAKE, FAKE,
                                                                    FAKE, None)]))
    assert call(bad) == 1                                       # the last layer is checked too
    assert call(arr, ws=16) == 6


def test_workspace_layout_prefill_and_decode():
    d = _desc(B=2, T=100, D=128, H=4, H_kv=2, d_h=64)
    L = lib.workspace_layout(d, 0)
    assert L.T_pad == 128
    esz, n_qkv = 2, (4 + 4) * 64
    assert L.q >= 2 * 100 * n_qkv * esz and L.q % 256 == 0
    assert L.k >= L.q + 2 * 4 * 100 * 64 * esz
    assert L.vt >= L.k + 2 * 2 * 128 * 64 * esz
    assert L.total_bytes >= L.vt + 2 * 2 * 64 * 128 * esz
    dd = _desc(B=16, T=1, D=3840, H=16, H_kv=8, d_h=256, attn_type="GLOBAL", window=0)
    Ld = lib.workspace_layout(dd, 131072)
    assert Ld.n_chunks * Ld.chunk >= 131072
    assert (3840 // 32) % Ld.ksplit_qkv == 0 and (4096 // 32) % Ld.ksplit_out == 0
    dl = _desc(B=16, T=1, D=3840, H=16, H_kv=8, d_h=256, window=1024)
    Ll = lib.workspace_layout(dl, 131072)
    assert Ll.n_chunks * Ll.chunk >= 1024 and Ll.total_bytes < Ld.total_bytes


def test_static_decode_refuses_before_any_device_call():
    # the allocation-free decode checks its workspace need against the
    # static scratch before touching the device: 27B-shaped rows at full
    # cache length need 300 MiB (scratch error), invalid shapes keep their
    # own status; no GPU is needed for either
    big = _desc(B=128, T=1, D=5376, H=32, H_kv=16, d_h=128, attn_type="GLOBAL", window=0)
    assert lib.workspace_bytes(big, 131072) > lib.STATIC_SCRATCH_BYTES
    w = lib.Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    f = lib._lib.gemma3_attn_decode_static
    assert f(ctypes.byref(big), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, 131072, FAKE, None) == 10
    assert f(ctypes.byref(big), FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, 0, FAKE, None) == 2
    assert f(None, FAKE, FAKE, ctypes.byref(w), FAKE, FAKE, 0, FAKE, None) == 1
    fits = _desc(B=16, T=1, D=3840, H=16, H_kv=8, d_h=256, attn_type="GLOBAL", window=0)
    assert lib.workspace_bytes(fits, 131072) <= lib.STATIC_SCRATCH_BYTES
    assert lib.STATUS[10] == "ERR_SCRATCH"
