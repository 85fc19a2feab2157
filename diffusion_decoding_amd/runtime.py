"""Torch-facing wrappers over the C ABI: device memory and streams come from
torch, every step of the path runs in libdg.so.  Nothing here computes."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (DG_DTYPE_BF16, DG_DTYPE_E8M0, DG_DTYPE_FP8_E4M3, DG_DTYPE_FP32, DG_DTYPE_MXFP4,
                   DG_DTYPE_MXFP4_MXFP8, dg_canvas, dg_config, dg_kv, dg_layer_weights, dg_step_out, dg_weights)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


_DT = {"fp32": DG_DTYPE_FP32, "bf16": DG_DTYPE_BF16, "fp8": DG_DTYPE_FP8_E4M3, "mxfp4": DG_DTYPE_MXFP4,
       "mxfp4_a8": DG_DTYPE_MXFP4_MXFP8, "e8m0": DG_DTYPE_E8M0}


def make_config(cfg) -> dg_config:
    return dg_config(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.head_dim, cfg.n_experts, cfg.top_k,
                     cfg.d_expert, cfg.d_shared, cfg.vocab, cfg.canvas_len, cfg.max_steps,
                     float(cfg.rope_theta), float(cfg.rms_eps), float(cfg.threshold),
                     _DT[cfg.act_dtype], _DT[cfg.expert_dtype], int(cfg.mask_token),
                     int(getattr(cfg, "self_condition", False)))


def pack_experts(w: torch.Tensor, dtype: str, stream=None) -> torch.Tensor:
    """Tiled copy (dg_pack_experts) of row-major expert matrices w[n][rows][cols]
    (bf16; fp8 codes as uint8; mxfp4 codes, two per uint8; e8m0: the mxfp4
    block scales [n][rows][K/32])."""
    if w.dim() != 3:
        raise ValueError("expert weights must be [n][rows][cols]")
    cols = w.shape[2] * {"mxfp4": 2, "e8m0": 32}.get(dtype, 1)   # codes per row
    out = torch.empty_like(w)
    _lib.dg_pack_experts(_ptr(w), _ptr(out), w.shape[0], w.shape[1], cols, _DT[dtype], _stream(stream))
    return out


class Model:
    """A libdg model over the weights of an ``Inputs`` set (tensors stay referenced)."""

    def __init__(self, inputs, max_batch: Optional[int] = None, max_tokens: Optional[int] = None,
                 max_kv: Optional[int] = None):
        cfg = inputs.cfg
        self.cfg = cfg
        self.inputs = inputs
        L = cfg.n_layers
        self._layers = (dg_layer_weights * L)()
        # bf16/fp8 routed experts go to the library in its tiled layout: one
        # packed copy per matrix, made here once and kept alive with the model
        self._packed = []
        for l, lw in enumerate(inputs.layers):
            w_gu, w_d, s_gu, s_d = lw["w_gu"], lw["w_d"], lw.get("s_gu"), lw.get("s_d")
            if cfg.expert_dtype != "fp32":
                pdt = "mxfp4" if cfg.expert_dtype == "mxfp4_a8" else cfg.expert_dtype   # same weight layout
                w_gu, w_d = pack_experts(w_gu, pdt), pack_experts(w_d, pdt)
                self._packed += [w_gu, w_d]
            if cfg.expert_dtype in ("mxfp4", "mxfp4_a8"):
                s_gu, s_d = pack_experts(s_gu, "e8m0"), pack_experts(s_d, "e8m0")
                self._packed += [s_gu, s_d]
            self._layers[l] = dg_layer_weights(
                _ptr(lw["wqkv"]), _ptr(lw["wo"]), _ptr(lw["wr"]), _ptr(w_gu), _ptr(w_d),
                _ptr(s_gu), _ptr(s_d), _ptr(lw["ws_gu"]), _ptr(lw["ws_d"]),
                _ptr(lw.get("ss_gu")), _ptr(lw.get("ss_d")))
        self._weights = dg_weights(_ptr(inputs.embed), _ptr(inputs.lm_head), self._layers)
        self._cfg = make_config(cfg)
        self.max_batch = max_batch or cfg.batch
        self.max_tokens = max_tokens or max(cfg.canvas_len, cfg.prompt_len if cfg.prompt_mode == "tokens" else 0)
        self.max_kv = max_kv or inputs.kv_k.shape[3]
        self.handle = _lib.dg_model_create(self._cfg, self._weights, self.max_batch, self.max_tokens,
                                           self.max_kv)

    def close(self):
        if self.handle is not None and self.handle.value:
            _lib.dg_model_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass
class Canvas:
    tokens: torch.Tensor      # int32 [B, N]
    committed: torch.Tensor   # uint8 [B, N]
    seed: int
    block: int = 0
    step: int = 0
    prediction: Optional[torch.Tensor] = None  # int32 [B, N]: previous step's argmax (self-conditioning)

    @classmethod
    def empty(cls, batch: int, n: int, seed: int, block: int = 0, device="cuda"):
        return cls(torch.zeros(batch, n, dtype=torch.int32, device=device),
                   torch.zeros(batch, n, dtype=torch.uint8, device=device), seed, block, 0,
                   torch.zeros(batch, n, dtype=torch.int32, device=device))

    def struct(self) -> dg_canvas:
        return dg_canvas(_ptr(self.tokens), _ptr(self.committed), self.tokens.shape[0], self.step,
                         self.seed, self.block, _ptr(self.prediction))


@dataclass
class KVCache:
    k: torch.Tensor   # [L, B, H, cap, dh]
    v: torch.Tensor
    length: int

    def struct(self) -> dg_kv:
        return dg_kv(_ptr(self.k), _ptr(self.v), self.k.shape[1], self.k.shape[3], self.length)


def canvas_init(model: Model, canvas: Canvas, stream=None):
    s = canvas.struct()
    _lib.dg_canvas_init(model.handle, s, _stream(stream))
    canvas.step = s.step


def canvas_prefill(model: Model, canvas: Canvas, tokens: torch.Tensor, mask: torch.Tensor, stream=None):
    """Pre-commit the positions where ``mask`` (uint8 [B, N]) is set to ``tokens``
    (int32 [B, N]); after canvas_init, before the first step."""
    B, N = canvas.tokens.shape
    if tuple(tokens.shape) != (B, N) or tuple(mask.shape) != (B, N):
        raise ValueError(f"tokens/mask must be [{B}, {N}]")
    if tokens.dtype != torch.int32 or mask.dtype != torch.uint8:
        raise TypeError("tokens must be int32 and mask uint8")
    if not (tokens.is_cuda and mask.is_cuda and tokens.is_contiguous() and mask.is_contiguous()):
        raise ValueError("tokens and mask must be contiguous device tensors")
    s = canvas.struct()
    _lib.dg_canvas_prefill(model.handle, s, _ptr(tokens), _ptr(mask), _stream(stream))


def denoise_step(model: Model, canvas: Canvas, kv: KVCache, entropy=None, argmax=None, top2_gap=None,
                 n_uncommitted=None, logits=None, hidden=None, status=None, expert_counts=None, stream=None):
    s = canvas.struct()
    out = dg_step_out(_ptr(entropy), _ptr(argmax), _ptr(top2_gap), _ptr(n_uncommitted), _ptr(logits),
                      _ptr(hidden), _ptr(status), _ptr(expert_counts))
    _lib.dg_denoise_step(model.handle, s, kv.struct(), out, _stream(stream))
    canvas.step = s.step


def generate_canvas(model: Model, canvas: Canvas, kv: KVCache, stream=None) -> int:
    s = canvas.struct()
    try:
        return _lib.dg_generate_canvas(model.handle, s, kv.struct(), _stream(stream))
    finally:
        canvas.step = s.step   # steps that ran before an error still count


def commit_canvas(model: Model, tokens: torch.Tensor, kv: KVCache, stream=None):
    if tokens.dtype != torch.int32 or tokens.dim() != 2:
        raise ValueError("tokens must be int32 [batch, n]")
    if tokens.shape[0] != kv.k.shape[1]:
        raise ValueError(f"tokens hold {tokens.shape[0]} canvases, the KV cache {kv.k.shape[1]}")
    s = kv.struct()
    _lib.dg_commit_canvas(model.handle, _ptr(tokens), tokens.shape[1], s, _stream(stream))
    kv.length = s.length


@dataclass
class Append:
    """A causal pass of a mixed batch: ``tokens`` (int32 [n], device) appended
    to the batch-1 cache ``kv`` (a prompt read or a committed canvas)."""
    kv: KVCache
    tokens: torch.Tensor


@dataclass
class Refine:
    """One denoise step of a batch-1 canvas in a mixed batch; the optional
    outputs are device tensors of [canvas_len] (entropy fp32, argmax int32)
    and [1] (n_uncommitted int32)."""
    kv: KVCache
    canvas: Canvas
    entropy: Optional[torch.Tensor] = None
    argmax: Optional[torch.Tensor] = None
    n_uncommitted: Optional[torch.Tensor] = None
    hidden: Optional[torch.Tensor] = None   # diagnostic: final normed hidden [canvas_len, d_model]


def mixed_step(model: Model, segments, status=None, stream=None):
    """One pass over requests in different phases (Append and Refine items),
    each with its own batch-1 cache; updates canvas.step and kv.length."""
    segs = list(segments)
    n_segs = len(segs)
    arr = (_lib.dg_segment * max(n_segs, 1))()
    keep = []
    for i, g in enumerate(segs):
        if g.kv.k.shape[1] != 1:
            raise ValueError(f"segment {i}: a mixed batch takes batch-1 caches")
        kvs = g.kv.struct()
        keep.append(kvs)
        if isinstance(g, Append):
            t = g.tokens
            if t.dtype != torch.int32 or t.dim() != 1 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"segment {i}: tokens must be a contiguous int32 device vector")
            arr[i] = _lib.dg_segment(_lib.DG_SEG_APPEND, t.shape[0], ctypes.pointer(kvs), _ptr(t), None,
                                     None, None, None, None)
        elif isinstance(g, Refine):
            if g.canvas.tokens.shape[0] != 1:
                raise ValueError(f"segment {i}: a refine segment holds one canvas")
            cs = g.canvas.struct()
            keep.append(cs)
            arr[i] = _lib.dg_segment(_lib.DG_SEG_REFINE, g.canvas.tokens.shape[1], ctypes.pointer(kvs), None,
                                     ctypes.pointer(cs), _ptr(g.entropy), _ptr(g.argmax), _ptr(g.n_uncommitted),
                                     _ptr(g.hidden))
        else:
            raise TypeError(f"segment {i}: {type(g).__name__} is neither Append nor Refine")
    _lib.dg_mixed_step(model.handle, arr, n_segs, _ptr(status), _stream(stream))
    for i, g in enumerate(segs):
        g.kv.length = arr[i].kv.contents.length
        if isinstance(g, Refine):
            g.canvas.step = arr[i].canvas.contents.step


def test_philox(seed, pos0, tag, canvas, block, modulus, n, stream=None) -> torch.Tensor:
    out = torch.empty(n, dtype=torch.int64, device="cuda")
    buf = torch.empty(n, dtype=torch.int32, device="cuda")
    _lib.dg_test_philox(seed, pos0, tag, canvas, block, modulus, n, _ptr(buf), _stream(stream))
    out.copy_(buf.to(torch.int64) & 0xFFFFFFFF)
    return out


def test_lm_head(model: Model, hf: torch.Tensor, stream=None):
    T = hf.shape[0]
    ent = torch.empty(T, dtype=torch.float32, device=hf.device)
    am = torch.empty(T, dtype=torch.int32, device=hf.device)
    gap = torch.empty(T, dtype=torch.float32, device=hf.device)
    _lib.dg_test_lm_head(model.handle, _ptr(hf), T, _ptr(ent), _ptr(am), _ptr(gap), _stream(stream))
    return ent, am, gap


def lm_head_confidence_noalloc(model: Model, hf: torch.Tensor, entropy: torch.Tensor, argmax: torch.Tensor,
                               top2_gap: Optional[torch.Tensor] = None, stream=None):
    """The allocation-free LM head + confidence: outputs are the caller's tensors."""
    _lib.dg_lm_head_confidence_noalloc(model.handle, _ptr(hf), hf.shape[0], _ptr(entropy), _ptr(argmax),
                                       _ptr(top2_gap), _stream(stream))


def test_commit(model: Model, canvas: Canvas, entropy: torch.Tensor, argmax: torch.Tensor, stream=None):
    nunc = torch.empty(canvas.tokens.shape[0], dtype=torch.int32, device=entropy.device)
    _lib.dg_test_commit(model.handle, canvas.struct(), _ptr(entropy), _ptr(argmax), _ptr(nunc),
                        _stream(stream))
    return nunc


# ---- unit entries (tests): one phase of a block on given buffers

def _dt(model: Model):
    return torch.bfloat16 if model.cfg.act_dtype == "bf16" else torch.float32


def test_qkv_rope(model: Model, layer: int, a: torch.Tensor, batch: int, pos0: int, stream=None):
    cfg = model.cfg
    n = a.shape[0] // batch
    shp = (batch, cfg.n_heads, n, cfg.head_dim)
    q, k, v = (torch.empty(shp, dtype=_dt(model), device=a.device) for _ in range(3))
    _lib.dg_test_qkv_rope(model.handle, layer, _ptr(a), batch, n, pos0, _ptr(q), _ptr(k), _ptr(v),
                          _stream(stream))
    return q, k, v


def test_attention(model: Model, layer: int, q: torch.Tensor, kv: KVCache, k_canvas=None, v_canvas=None,
                   stream=None):
    B, H, n, dh = q.shape
    out = torch.empty(B * n, H * dh, dtype=_dt(model), device=q.device)
    _lib.dg_test_attention(model.handle, layer, _ptr(q), kv.struct(), _ptr(k_canvas), _ptr(v_canvas), n,
                           _ptr(out), _stream(stream))
    return out


def test_router(model: Model, layer: int, b: torch.Tensor, stream=None):
    cfg, T = model.cfg, b.shape[0]
    logits = torch.empty(T, cfg.n_experts, dtype=torch.float32, device=b.device)
    ids = torch.empty(T, cfg.top_k, dtype=torch.int32, device=b.device)
    w = torch.empty(T, cfg.top_k, dtype=torch.float32, device=b.device)
    _lib.dg_test_router(model.handle, layer, _ptr(b), T, _ptr(logits), _ptr(ids), _ptr(w), _stream(stream))
    return logits, ids, w


def test_shared(model: Model, layer: int, b: torch.Tensor, stream=None):
    cfg, T = model.cfg, b.shape[0]
    hs = torch.empty(T, cfg.d_shared, dtype=_dt(model), device=b.device)
    ys = torch.empty(T, cfg.d_model, dtype=torch.float32, device=b.device)
    _lib.dg_test_shared(model.handle, layer, _ptr(b), T, _ptr(hs), _ptr(ys), _stream(stream))
    return hs, ys


def test_moe(model: Model, layer: int, b: torch.Tensor, ids: torch.Tensor, stream=None):
    cfg, T = model.cfg, b.shape[0]
    if ids.dtype != torch.int32 or tuple(ids.shape) != (T, cfg.top_k):
        raise ValueError(f"ids must be int32 [{T}, {cfg.top_k}]")
    h = torch.empty(T * cfg.top_k, cfg.d_expert, dtype=_dt(model), device=b.device)
    y = torch.empty(T * cfg.top_k, cfg.d_model, dtype=torch.float32, device=b.device)
    pos = torch.empty(T, cfg.top_k, dtype=torch.int32, device=b.device)
    _lib.dg_test_moe(model.handle, layer, _ptr(b), T, _ptr(ids), _ptr(h), _ptr(y), _ptr(pos), _stream(stream))
    return h, y, pos


def test_force_routing(model: Model, ids: Optional[torch.Tensor]):
    """ids: int32 [n_layers, max_batch * canvas_len, top_k] (-1 rows: not forced), kept
    referenced by the model while set; None turns forcing off."""
    if ids is not None:
        cfg = model.cfg
        want = (cfg.n_layers, model.max_batch * cfg.canvas_len, cfg.top_k)
        if ids.dtype != torch.int32 or tuple(ids.shape) != want:
            raise ValueError(f"ids must be int32 {want}")
    model._forced = ids
    _lib.dg_test_force_routing(model.handle, _ptr(ids))


def test_mx8_quantize(x: torch.Tensor, norm_eps: Optional[float] = None, stream=None):
    """bf16 rows x [rows][d] -> (codes uint8 [rows][d], scales uint8 [rows][d/32], y): the MXFP8
    rows the MXFP4 x MXFP8 experts read; with norm_eps, of y = bf16(rmsnorm(x)) (else y is None)."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("need contiguous bf16 [rows][d]")
    rows, d = x.shape
    codes = torch.empty(rows, d, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, d // 32, dtype=torch.uint8, device=x.device)
    y = torch.empty_like(x) if norm_eps is not None else None
    _lib.dg_test_mx8_quantize(_ptr(x), rows, d, int(norm_eps is not None), float(norm_eps or 0.0),
                              _ptr(y), _ptr(codes), _ptr(scales), _stream(stream))
    return codes, scales, y


def test_fp4_decode(packed: torch.Tensor, scales: torch.Tensor, stream=None) -> torch.Tensor:
    """packed uint8 [n_blocks * 16], scales uint8 [n_blocks] -> bf16 [n_blocks * 32]."""
    nb = scales.numel()
    if packed.numel() != 16 * nb or packed.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise ValueError("need uint8 packed [16 * n_blocks] and scales [n_blocks]")
    out = torch.empty(32 * nb, dtype=torch.bfloat16, device=packed.device)
    _lib.dg_test_fp4_decode(_ptr(packed), _ptr(scales), nb, _ptr(out), _stream(stream))
    return out
