"""Seeded generator of synthetic inputs.

Recipe (one independent torch.Generator per tensor, seeded from the workload
seed and the tensor's ordinal, on the device the run uses):

* token embedding ``embed[V, d] ~ N(0, 1)`` (untied from the LM head);
* every projection ``W[out, in] ~ N(0, 1/in)`` (``in`` = fan-in), stored in the
  ``[out][in]`` layout: wqkv ``[3*H*dh, d]`` (q rows, then k, then v), wo
  ``[d, H*dh]``, router wr ``[E, d]``, routed experts ``w_gu[E, 2*de, d]`` (gate
  rows then up rows) and ``w_d[E, d, de]``, shared expert ``ws_gu[2*ds, d]`` and
  ``ws_d[d, ds]``;
* LM head ``lm_head[V, d] ~ N(0, 1/d) * lm_scale``;
* prompt KV cache ``kv_k, kv_v[L, B, H, cap, dh]``: rows ``[0, P)`` ~ N(0, 1),
  already rotary-embedded; the rest zero;
* for block-autoregressive runs, prompt token ids uniform on ``[0, V)``.

Values are drawn in fp32 and cast to the storage type (``bf16``: round to
nearest even).  fp8 expert weights are OCP E4M3FN codes with one fp32 scale per
output channel, ``scale = max|W[c, :]| / 448``, codes = RNE(W / scale) clamped
to +-448; the codes and scales are the inputs both sides receive.  mxfp4
routed-expert weights follow the OCP Microscaling conversion: each block of 32
consecutive weights along the input dimension gets the scale 2^e with
e = floor(log2(max|block|)) - 2 (2 is the largest E2M1 exponent), stored as the
E8M0 code e + 127 (an all-zero block gets code 0), and each weight becomes the
E2M1 code nearest to w / 2^e (ties to the even mantissa, magnitudes above 6
saturate); two codes per byte, the even element in the low nibble.  The shared
expert stays bf16 in mxfp4 workloads.  mxfp4_a8 workloads draw the same
weights as mxfp4 ones (their activations differ only inside the kernels).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

from .configs import Config

_FP8_MAX = 448.0


def _gen(device, seed: int, ordinal: int) -> torch.Generator:
    g = torch.Generator(device=device)
    # SplitMix-style mix of (seed, ordinal) into a 63-bit torch seed.
    z = (seed * 0x9E3779B97F4A7C15 + (ordinal + 1) * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
    z ^= z >> 31
    z = (z * 0x94D049BB133111EB) & ((1 << 64) - 1)
    z ^= z >> 29
    g.manual_seed(z & ((1 << 63) - 1))
    return g


def _storage_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def _normal(shape, std, device, seed, ordinal, dtype):
    g = _gen(device, seed, ordinal)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def quantize_fp8_rows(w32: torch.Tensor):
    """Per-output-channel E4M3FN quantization of ``w32[..., out, in]``."""
    amax = w32.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    scale = (amax / _FP8_MAX).to(torch.float32)
    q = (w32 / scale).clamp_(-_FP8_MAX, _FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.squeeze(-1).contiguous()


# E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (code = index): the midpoints
# between neighbours, and which midpoints round up (to an even mantissa)
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_TIE_UP = (False, True, False, True, False, True, False)


def quantize_mxfp4_rows(w32: torch.Tensor):
    """MXFP4 quantization of ``w32[..., K]`` (K % 32 == 0) in blocks of 32 along
    the last axis: returns (packed codes uint8 [..., K/2], E8M0 scales uint8
    [..., K/32])."""
    *lead, K = w32.shape
    blk = w32.reshape(*lead, K // 32, 32).to(torch.float32)
    amax = blk.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-38))) - 2, torch.full_like(amax, -127.0))
    e = e.clamp(-127, 127)
    v = blk / torch.exp2(e)[..., None]
    a = v.abs()
    mid = torch.tensor(_E2M1_MID, dtype=torch.float32, device=w32.device)
    idx = torch.bucketize(a, mid)                       # midpoints strictly below |v|
    for j, up in enumerate(_E2M1_TIE_UP):
        if up:
            idx = torch.where(a == mid[j], torch.full_like(idx, j + 1), idx)
    codes = (idx | torch.where(v < 0, 8, 0)).to(torch.uint8).reshape(*lead, K)
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


@dataclass
class Inputs:
    cfg: Config
    embed: torch.Tensor
    lm_head: torch.Tensor
    layers: list
    kv_k: torch.Tensor
    kv_v: torch.Tensor
    kv_len: int
    prompt_tokens: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)

    @property
    def device(self):
        return self.embed.device


def _expert_tensor(shape, fan_in, cfg, device, ordinal, dtype, routed=True):
    """Returns (weights, scales-or-None) in the expert storage format."""
    std = fan_in ** -0.5
    if cfg.expert_dtype in ("mxfp4", "mxfp4_a8") and routed:
        g = _gen(device, cfg.seed, ordinal)
        w32 = torch.randn(*shape, generator=g, device=device, dtype=torch.float32).mul_(std)
        q, s = quantize_mxfp4_rows(w32)
        del w32
        return q, s
    if cfg.expert_dtype in ("mxfp4", "mxfp4_a8"):
        return _normal(shape, std, device, cfg.seed, ordinal, dtype), None
    if cfg.expert_dtype == "fp8":
        g = _gen(device, cfg.seed, ordinal)
        w32 = torch.randn(*shape, generator=g, device=device, dtype=torch.float32).mul_(std)
        q, s = quantize_fp8_rows(w32)
        del w32
        return q, s
    return _normal(shape, std, device, cfg.seed, ordinal, dtype), None


def make_inputs(cfg: Config, device="cpu", kv_capacity: Optional[int] = None) -> Inputs:
    """Draw every input of workload ``cfg`` on ``device``."""
    device = torch.device(device)
    act = _storage_dtype(cfg.act_dtype)
    edt = torch.float32 if cfg.expert_dtype == "fp32" else torch.bfloat16  # fp8 / mxfp4: codes
    d, V = cfg.d_model, cfg.vocab
    ad = cfg.attn_dim
    E, de, ds = cfg.n_experts, cfg.d_expert, cfg.d_shared
    embed = _normal((V, d), 1.0, device, cfg.seed, 0, act)
    lm_head = _normal((V, d), cfg.lm_scale * d ** -0.5, device, cfg.seed, 1, act)
    layers = []
    for l in range(cfg.n_layers):
        base = 16 + 16 * l
        lw = {
            "wqkv": _normal((cfg.qkv_dim, d), d ** -0.5, device, cfg.seed, base + 0, act),
            "wo": _normal((d, ad), ad ** -0.5, device, cfg.seed, base + 1, act),
            "wr": _normal((E, d), d ** -0.5, device, cfg.seed, base + 2, act),
        }
        lw["w_gu"], lw["s_gu"] = _expert_tensor((E, 2 * de, d), d, cfg, device, base + 3, edt)
        lw["w_d"], lw["s_d"] = _expert_tensor((E, d, de), de, cfg, device, base + 4, edt)
        lw["ws_gu"], lw["ss_gu"] = _expert_tensor((2 * ds, d), d, cfg, device, base + 5, edt, routed=False)
        lw["ws_d"], lw["ss_d"] = _expert_tensor((d, ds), ds, cfg, device, base + 6, edt, routed=False)
        layers.append(lw)
    cap = kv_capacity if kv_capacity is not None else cfg.kv_capacity
    shape = (cfg.n_layers, cfg.batch, cfg.n_heads, cap, cfg.head_dim)
    kv_k = torch.zeros(shape, dtype=act, device=device)
    kv_v = torch.zeros(shape, dtype=act, device=device)
    prompt_tokens = None
    kv_len = 0
    if cfg.prompt_mode == "kv":
        P = cfg.prompt_len
        for l in range(cfg.n_layers):
            kv_k[l, :, :, :P] = _normal((cfg.batch, cfg.n_heads, P, cfg.head_dim), 1.0,
                                        device, cfg.seed, 16 + 16 * l + 7, act)
            kv_v[l, :, :, :P] = _normal((cfg.batch, cfg.n_heads, P, cfg.head_dim), 1.0,
                                        device, cfg.seed, 16 + 16 * l + 8, act)
        kv_len = P
    else:
        g = _gen(device, cfg.seed, 2)
        prompt_tokens = torch.randint(0, V, (cfg.batch, cfg.prompt_len), generator=g,
                                      device=device, dtype=torch.int32)
    return Inputs(cfg=cfg, embed=embed, lm_head=lm_head, layers=layers, kv_k=kv_k, kv_v=kv_v,
                  kv_len=kv_len, prompt_tokens=prompt_tokens)
