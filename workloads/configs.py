"""Workload shapes for DiffusionGemma-style block diffusion decoding.

The backbone facts come from the pages on DiffusionGemma: a 256-token canvas
(DiffusionGemma解析, "整片并行去噪"; zhichai.net 深度拆解, "Block-Autoregressive"),
at most 48 denoise steps (DiffusionGemma解析, "自适应停步机制"), 128 experts with
top-8 routing plus one shared expert (zhichai.net 深度拆解, "MoE 效率"), and a
vocabulary of about 250K (DiffusionGemma解析, "自回归的瓶颈").  Everything the
pages leave open (layer width, heads, expert width, prompt length) is a
synthetic stand-in chosen to match those facts.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    d_expert: int
    d_shared: int
    vocab: int
    canvas_len: int
    max_steps: int
    prompt_len: int          # tokens already in the KV cache (random K,V) or prompt tokens (encoded)
    batch: int
    act_dtype: str           # "fp32" or "bf16"
    expert_dtype: str        # "fp32", "bf16", "fp8" (routed and shared), "mxfp4" or "mxfp4_a8" (routed; shared bf16)
    seed: int
    lm_scale: float = 1.0    # multiplies the N(0, 1/d) LM-head draw
    rope_theta: float = 1.0e4
    rms_eps: float = 1.0e-6
    threshold: float = 1.0   # nats; uncommitted positions below it commit at once
    n_canvases: int = 1      # canvases generated one after another (block-AR)
    prompt_mode: str = "kv"  # "kv": random post-RoPE K,V; "tokens": ids encoded by a causal pass
    mask_token: int = -1     # -1: uniform-state noise; a vocabulary id: absorbing-state ([MASK]) noise
    self_condition: bool = False  # each step after the first adds the embedding of the previous step's argmax

    @property
    def qkv_dim(self) -> int:
        return 3 * self.n_heads * self.head_dim

    @property
    def attn_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_capacity(self) -> int:
        """Rows of KV cache per (layer, canvas) needed by the whole workload."""
        if self.prompt_mode == "tokens":
            return self.prompt_len + self.n_canvases * self.canvas_len
        return self.prompt_len

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


_C0 = Config(
    name="c0_tiny_fp32", n_layers=1, d_model=64, n_heads=4, head_dim=16,
    n_experts=8, top_k=2, d_expert=32, d_shared=32, vocab=512,
    canvas_len=16, max_steps=8, prompt_len=32, batch=1,
    act_dtype="fp32", expert_dtype="fp32", seed=0, lm_scale=6.0,
)

_C1 = Config(
    name="c1_step_bf16", n_layers=1, d_model=2048, n_heads=16, head_dim=128,
    n_experts=128, top_k=8, d_expert=704, d_shared=2048, vocab=262144,
    canvas_len=256, max_steps=48, prompt_len=1024, batch=1,
    act_dtype="bf16", expert_dtype="bf16", seed=1,
)

_C2 = _C1.replace(name="c2_loop30_bf16", n_layers=30, prompt_len=2048, seed=2)

_C3 = _C2.replace(name="c3_batch4_p8192_bf16", batch=4, prompt_len=8192, seed=3)

_C4 = _C2.replace(name="c4_blockar_fp8", expert_dtype="fp8", prompt_len=512, seed=4,
                  n_canvases=8, prompt_mode="tokens")

# batch sweep beyond the four canvases of c3: eight canvases (2048 pooled
# expert tokens), each with its own 8192-row prompt KV cache
_C5 = _C3.replace(name="c5_batch8_p8192_bf16", batch=8, seed=5)

# the 30-layer loop with MXFP4 routed experts (OCP MX: E2M1 codes with one
# E8M0 scale per 32 weights; the pages' 4-bit experts are NVFP4 on NVIDIA
# parts -- DiffusionGemma深度拆解 (zhichai.net), "MoE 效率"), shared expert bf16
_C6 = _C2.replace(name="c6_loop30_mxfp4", expert_dtype="mxfp4", seed=6)
# the same weights with the routed gate/up inputs in MXFP8 (E4M3 elements, one
# E8M0 scale per 32), for gfx950's scaled MFMA on 4-bit x 8-bit operands
_C7 = _C6.replace(name="c7_loop30_mxfp4_a8", expert_dtype="mxfp4_a8")

CONFIGS = {c.name: c for c in (_C0, _C1, _C2, _C3, _C4, _C5, _C6, _C7)}
_ALIASES = {"c0": _C0.name, "c1": _C1.name, "c2": _C2.name, "c3": _C3.name, "c4": _C4.name,
            "c5": _C5.name, "c6": _C6.name, "c7": _C7.name}


def get_config(name: str) -> Config:
    return CONFIGS[_ALIASES.get(name, name)]


def tiny_config(**kw) -> Config:
    """A c0-shaped config with overrides, for unit tests."""
    kw.setdefault("name", "tiny")
    return _C0.replace(**kw)
