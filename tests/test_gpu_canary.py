"""Guard bands around every buffer the library writes. Each output y, each
workspace and each cache sits inside a larger allocation whose bytes before
and after it hold a fixed pattern; after the call (and a synchronize) the
pattern must be intact, so no kernel writes outside the buffers the C ABI
hands it (outputs, workspaces and caches are sized exactly as the ABI's size
functions and shape rules say). Shapes are ragged (T, D and valid lengths off
every tile size) and cover the split-KV prefill, the cache-filling prefill,
the chunk, decode, the block and the routed stack, bf16 and fp32."""

import ctypes

import numpy as np
import pytest
import torch

from workloads import inputs as I
from parity_util import log, small_prefill_inputs, to_dev, weights_of

pytestmark = pytest.mark.gpu

L, G = "LOCAL_SLIDING", "GLOBAL"
PAD = 4096  # bytes of guard band on each side (a multiple of 256: alignment is kept)
PATTERN = 0xA5


class Guarded:
    """A tensor of `shape` inside a buffer with PAD guard bytes on both sides."""

    def __init__(self, shape, dtype, fill=None):
        esz = torch.empty((), dtype=dtype).element_size()
        self.n = int(np.prod(shape)) * esz
        self.raw = torch.full((self.n + 2 * PAD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[PAD:PAD + self.n].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def check(self, what):
        torch.cuda.synchronize()
        head = self.raw[:PAD].cpu().numpy()
        tail = self.raw[PAD + self.n:].cpu().numpy()
        bad = int((head != PATTERN).sum() + (tail != PATTERN).sum())
        assert bad == 0, f"{what}: {bad} guard bytes overwritten"


def _kw(H, Hk, d_h, attn_type, window):
    return dict(H=H, H_kv=Hk, d_h=d_h, attn_type=attn_type, window=window,
                rope_theta=1e4 if attn_type == L else 1e6,
                rope_scale=1.0 if attn_type == L else 8.0, query_scale=d_h ** -0.5)


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


# B, T, D, H, H_kv, d_h, dtype, valid lengths (T = 200 on the 1B-like heads
# gives too few query tiles to fill the chip, so the key ranges are split)
CASES = [
    (2, 321, 256, 4, 2, 64, "bf16", (321, 200)),
    (1, 200, 1152, 4, 1, 256, "bf16", None),
    (1, 300, 512, 4, 2, 128, "bf16", None),
    (2, 150, 192, 2, 1, 64, "f32", (150, 77)),   # decode takes d_h in {64, 128, 256}
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
@pytest.mark.parametrize("attn_type,window", [(L, 100), (G, 0)])
def test_prefill_cache_chunk_decode_stay_inside(gpu_lib, case, attn_type, window):
    B, T, D, H, Hk, d_h, dtype, lens = case
    log(f"guard bands {case} {attn_type}")
    kw = _kw(H, Hk, d_h, attn_type, window)
    tdt = _tdt(dtype)
    d = to_dev(small_prefill_inputs(61, B, T, D, H, Hk, d_h, dtype, lens))
    desc = gpu_lib.make_desc(B=B, T=T, D=D, dtype=tdt, **kw)
    kvl = d["kv_valid_len"]

    # plain prefill
    y = Guarded((B, T, D), tdt)
    ws = Guarded((gpu_lib.workspace_bytes(desc),), torch.uint8)
    gpu_lib.prefill(d["x"], d["segment_pos"], weights_of(d), kv_valid_len=kvl, workspace=ws.t,
                    y=y.t, **kw)
    y.check("prefill y")
    ws.check("prefill workspace")

    # cache-filling prefill of the first part, then a chunk of the rest
    S = T + 37
    cut = T // 2 + 3
    kc = Guarded((B, S, Hk, d_h), tdt, float("nan"))
    vc = Guarded((B, S, Hk, d_h), tdt, float("nan"))
    first = {k: v for k, v in d.items()}
    first.update(x=d["x"][:, :cut].contiguous(), segment_pos=d["segment_pos"][:, :cut].contiguous())
    desc1 = gpu_lib.make_desc(B=B, T=cut, D=D, dtype=tdt, **kw)
    y1 = Guarded((B, cut, D), tdt)
    ws1 = Guarded((gpu_lib.workspace_bytes(desc1),), torch.uint8)
    gpu_lib.prefill(first["x"], first["segment_pos"], weights_of(d), workspace=ws1.t, y=y1.t,
                    k_cache=kc.t, v_cache=vc.t, **kw)
    for g, what in ((y1, "cache prefill y"), (ws1, "cache prefill workspace"),
                    (kc, "k cache"), (vc, "v cache")):
        g.check(what)
    Tc = T - cut
    descc = gpu_lib.make_desc(B=B, T=Tc, D=D, dtype=tdt, **kw)
    n = gpu_lib._lib.gemma3_attn_prefill_chunk_workspace_bytes(ctypes.byref(descc), cut)
    wsc = Guarded((n,), torch.uint8)
    yc = Guarded((B, Tc, D), tdt)
    clen = None if kvl is None else torch.clamp(kvl - cut, min=1).to(torch.int32)
    gpu_lib.prefill_chunk(d["x"][:, cut:].contiguous(), d["segment_pos"][:, cut:].contiguous(),
                          weights_of(d), kc.t, vc.t, cut, kv_valid_len=clen, workspace=wsc.t,
                          y=yc.t, **kw)
    for g, what in ((yc, "chunk y"), (wsc, "chunk workspace"), (kc, "k cache"),
                    (vc, "v cache")):
        g.check(what)

    # decode one token per row at the slot after its last valid one
    r = np.random.default_rng([62, B, D])
    xt = I.to_dtype(r.standard_normal((B, 1, D)), dtype).cuda()
    pos = (torch.full((B,), T, dtype=torch.int32, device="cuda") if clen is None
           else (cut + clen).to(torch.int32)).reshape(B, 1).contiguous()
    descd = gpu_lib.make_desc(B=B, T=1, D=D, dtype=tdt, **kw)
    wsd = Guarded((gpu_lib.workspace_bytes(descd, S),), torch.uint8)
    yd = Guarded((B, 1, D), tdt)
    gpu_lib.decode(xt, pos, weights_of(d), kc.t, vc.t, workspace=wsd.t, y=yd.t, **kw)
    for g, what in ((yd, "decode y"), (wsd, "decode workspace"), (kc, "k cache"),
                    (vc, "v cache")):
        g.check(what)
    assert torch.isfinite(yd.t.float()).all()


def _block_weights(seed, D, H, Hk, d_h, D_ff, dtype):
    r = np.random.default_rng([seed, D, D_ff])
    std = D ** -0.5
    w = dict(w_q=r.standard_normal((H * d_h, D)) * std,
             w_kv=r.standard_normal((2 * Hk * d_h, D)) * std,
             w_o=r.standard_normal((D, H * d_h)) * std,
             gamma_q=r.standard_normal(d_h) * 0.1, gamma_k=r.standard_normal(d_h) * 0.1,
             w_gating=r.standard_normal((2, D_ff, D)) * std,
             w_linear=r.standard_normal((D, D_ff)) * D_ff ** -0.5)
    for k in ("pre_attn_norm", "post_attn_norm", "pre_ffw_norm", "post_ffw_norm"):
        w[k] = r.standard_normal(D) * 0.1
    return {k: I.to_dtype(v, dtype).cuda() for k, v in w.items()}


@pytest.mark.parametrize("dtype,d_h", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_block_and_stack_stay_inside(gpu_lib, dtype, d_h):
    B, T, H, Hk, D_ff, Wn, S, n = 2, 150, 4, 2, 320, 48, 190, 7
    D = H * d_h
    log(f"guard bands block/stack {dtype} d_h={d_h}")
    tdt = _tdt(dtype)
    d = to_dev(small_prefill_inputs(63, B, T, D, H, Hk, d_h, dtype, (150, 111)))
    layers = [_block_weights(64 + l, D, H, Hk, d_h, D_ff, dtype) for l in range(n)]
    kw = _kw(H, Hk, d_h, L, Wn)
    desc = gpu_lib.make_desc(B=B, T=T, D=D, dtype=tdt, **kw)

    y = Guarded((B, T, D), tdt)
    ws = Guarded((gpu_lib._lib.gemma3_block_workspace_bytes(ctypes.byref(desc), D_ff),),
                 torch.uint8)
    gpu_lib.block_prefill(d["x"], d["segment_pos"], dict(d, **layers[0]),
                          kv_valid_len=d["kv_valid_len"], workspace=ws.t, y=y.t, **kw)
    y.check("block y")
    ws.check("block workspace")

    kc = Guarded((B, S, Hk, d_h), tdt, float("nan"))
    vc = Guarded((B, S, Hk, d_h), tdt, float("nan"))
    r = np.random.default_rng([65, D])
    xt = I.to_dtype(r.standard_normal((B, 1, D)), dtype).cuda()
    pos = torch.tensor([[5], [17]], dtype=torch.int32, device="cuda")
    descd = gpu_lib.make_desc(B=B, T=1, D=D, dtype=tdt, **kw)
    wsd = Guarded((gpu_lib._lib.gemma3_block_decode_workspace_bytes(ctypes.byref(descd), D_ff, S),),
                  torch.uint8)
    yd = Guarded((B, 1, D), tdt)
    kc.t.zero_()
    vc.t.zero_()
    gpu_lib.block_decode(xt, pos, layers[0], kc.t, vc.t, workspace=wsd.t, y=yd.t, **kw)
    for g, what in ((yd, "block decode y"), (wsd, "block decode workspace"), (kc, "k cache"),
                    (vc, "v cache")):
        g.check(what)

    skw = dict(H=H, H_kv=Hk, d_h=d_h, window=Wn, query_scale=d_h ** -0.5,
               local_rope=(1e4, 1.0), global_rope=(1e6, 8.0))
    kcs = [Guarded((B, S, Hk, d_h), tdt, float("nan")) for _ in range(n)]
    vcs = [Guarded((B, S, Hk, d_h), tdt, float("nan")) for _ in range(n)]
    ys = Guarded((B, T, D), tdt)
    gpu_lib.stack_prefill(d["x"], d["segment_pos"], layers, kv_valid_len=d["kv_valid_len"],
                          k_caches=[g.t for g in kcs], v_caches=[g.t for g in vcs], y=ys.t, **skw)
    ys.check("stack y")
    for l in range(n):
        kcs[l].check(f"layer {l} k cache")
        vcs[l].check(f"layer {l} v cache")
    pos = d["kv_valid_len"].to(torch.int32).reshape(B, 1)
    ysd = Guarded((B, 1, D), tdt)
    gpu_lib.stack_decode(xt, pos, layers, [g.t for g in kcs], [g.t for g in vcs], y=ysd.t, **skw)
    ysd.check("stack decode y")
    for l in range(n):
        kcs[l].check(f"decode layer {l} k cache")
        vcs[l].check(f"decode layer {l} v cache")
    assert torch.isfinite(ysd.t.float()).all()


def test_guard_check_sees_a_stray_byte():
    # the checker itself: one byte changed just outside the buffer (by torch,
    # not by a kernel of the library) must be reported, on either side
    for where in ("head", "tail"):
        g = Guarded((3, 5), torch.bfloat16)
        g.raw[PAD - 1 if where == "head" else PAD + g.n] = 0
        with pytest.raises(AssertionError):
            g.check(where)
