"""Denoise step, denoise loop and causal commit pass (test infrastructure only).

A plain float64 NumPy statement of what the block-diffusion decoder computes.
Pages (four DiffusionGemma write-ups) and the passages each function follows:

* DiffusionGemma解析, section "换个路数：整片并行去噪的生成机制": a 256-slot canvas
  starts from random tokens; every round scores all positions at once, a
  per-position distribution whose entropy measures confidence; positions are
  ranked from low to high entropy, the most certain are frozen and the rest
  are re-noised; attention over the canvas is bidirectional (no causal mask).
* DiffusionGemma解析, section "自适应停步机制": at most 48 steps per generation.
* zhichai.net 深度拆解, "架构解剖": the prompt is read into a KV cache by a causal
  pass; the canvas attends bidirectionally; "Block-Autoregressive": canvases
  run in series and each finished canvas is encoded and appended to the KV
  cache; "双向注意力": canvas K/V are recomputed every step; "MoE 效率": 128
  fine-grained experts plus one shared expert, top-8 routing; "统一状态扩散":
  uniform-state noise (no mask token).
* ipcmen.com, "工作原理：并行精炼与自我修正": each step locks the most confident
  tokens and randomises the uncertain positions for the next step.
* openai-hub.com (Google DeepMind 发布 DiffusionGemma), "为什么扩散能跑得比自回归快":
  self-conditioning is one of the techniques the model brings together (named
  only).  Reading, as an option of the config: every step after the first
  also feeds the model its own previous prediction -- the argmax at each
  position, the value the commit rule would lock -- by adding that token's
  embedding row to the position's input embedding (one sum, rounded once to
  the activation precision); the first step adds nothing.

Readings where the pages are silent (each is also listed in the design notes):
pre-norm RMSNorm blocks without gains and with a final norm before the LM head;
rotate-half RoPE at absolute positions ``P + i``; multi-head attention scaled by
``1/sqrt(dh)``; router softmax, top-k on the router logits (ties to the lower
expert id) renormalised over the k picks; SwiGLU experts; the shared expert
added with weight 1; the commit count ``m = ceil(U / (S_max - s))`` with 0-based
``s``, unioned with every uncommitted position whose entropy is below the
threshold; argmax commit value (lowest token id on ties); uniform re-noise with
Philox4x32-10.

Precision: ``fp32`` workloads are computed here in float64 without rounding.
``bf16`` workloads round to bfloat16 exactly where the GPU stores activations:
embedding rows, RMSNorm outputs, q/k/v (before and after RoPE), attention
output, each residual update (one rounding per add), and the SwiGLU product of
each expert.  Decisions taken from floating point (router top-k, argmax,
entropy ranking and threshold) are taken on values rounded to binary32, the
precision the GPU decides in.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np
import torch

from . import philox
from .numerics import decode_e4m3fn, decode_mxfp4, round_bf16, round_fp32, round_mxfp8


# ----------------------------------------------------------------------------- precision

class Prec:
    def __init__(self, act_dtype: str):
        self.bf16 = act_dtype == "bf16"

    def act(self, x):
        return round_bf16(x) if self.bf16 else x


# ----------------------------------------------------------------------------- weights

def _np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def _dequant(codes: torch.Tensor, scales: torch.Tensor) -> np.ndarray:
    q = decode_e4m3fn(codes.detach().to("cpu").numpy())
    s = scales.detach().to("cpu").to(torch.float64).numpy()
    return q * s[..., None]


class Weights:
    """float64 host views of an ``Inputs`` weight set, converted on demand."""

    def __init__(self, inputs, cache: bool = False):
        self.inp = inputs
        self.cfg = inputs.cfg
        self._cache = {} if cache else None
        self._embed_host = None

    def _get(self, key, fn):
        if self._cache is None:
            return fn()
        if key not in self._cache:
            self._cache[key] = fn()
        return self._cache[key]

    def embed_table(self) -> torch.Tensor:
        """Host copy of the embedding table (made once; every gather runs on the CPU)."""
        if self._embed_host is None:
            self._embed_host = self.inp.embed.detach().to("cpu")
        return self._embed_host

    def embed_rows(self, tok) -> np.ndarray:
        idx = torch.from_numpy(np.asarray(tok, dtype=np.int64).reshape(-1))
        return _np64(self.embed_table().index_select(0, idx)).reshape(*np.shape(tok), -1)

    def prefetch(self, layers: int):
        """Convert the weights of the first ``layers`` layers, the LM head and the
        embedding table ahead of time (needs ``cache=True``), so that a timed
        oracle run measures its arithmetic, not the weight conversion."""
        if self._cache is None:
            raise ValueError("prefetch needs a caching Weights (cache=True)")
        self.embed_table()
        for l in range(layers):
            for name in ("wqkv", "wo", "wr", "ws_gu", "ws_d"):
                self.dense(l, name)
            for e in range(self.cfg.n_experts):
                self.expert(l, e)
        for _ in self.lm_head_chunks():
            pass

    def lm_head_chunks(self, chunk: int = 16384):
        V = self.cfg.vocab
        for c0 in range(0, V, chunk):
            c1 = min(V, c0 + chunk)
            yield c0, c1, self._get(("lm", c0), lambda: _np64(self.inp.lm_head[c0:c1]))

    def dense(self, l: int, name: str) -> np.ndarray:
        lw = self.inp.layers[l]
        scale_name = {"ws_gu": "ss_gu", "ws_d": "ss_d"}.get(name)
        if scale_name and lw.get(scale_name) is not None:
            return self._get((l, name), lambda: _dequant(lw[name], lw[scale_name]))
        return self._get((l, name), lambda: _np64(lw[name]))

    def expert(self, l: int, e: int):
        lw = self.inp.layers[l]

        def load():
            if self.cfg.expert_dtype in ("mxfp4", "mxfp4_a8"):
                host = lambda t: t.detach().to("cpu").numpy()
                return (decode_mxfp4(host(lw["w_gu"][e]), host(lw["s_gu"][e])),
                        decode_mxfp4(host(lw["w_d"][e]), host(lw["s_d"][e])))
            if lw.get("s_gu") is not None:
                return _dequant(lw["w_gu"][e], lw["s_gu"][e]), _dequant(lw["w_d"][e], lw["s_d"][e])
            return _np64(lw["w_gu"][e]), _np64(lw["w_d"][e])
        return self._get((l, "expert", e), load)


class KV:
    """Per-layer, per-canvas K/V cache rows, kept exactly (float64 or bfloat16 storage)."""

    def __init__(self, kv_k: torch.Tensor, kv_v: torch.Tensor, length: int, bf16: bool):
        dt = torch.bfloat16 if bf16 else torch.float64
        self.k = kv_k.detach().to("cpu").to(dt).clone()
        self.v = kv_v.detach().to("cpu").to(dt).clone()
        self.length = int(length)

    @property
    def capacity(self) -> int:
        return self.k.shape[3]

    def get(self, l: int, b: int, n: Optional[int] = None):
        n = self.length if n is None else n
        return self.k[l, b, :, :n].double().numpy(), self.v[l, b, :, :n].double().numpy()

    def put(self, l: int, b: int, start: int, k: np.ndarray, v: np.ndarray):
        n = k.shape[1]
        self.k[l, b, :, start:start + n] = torch.from_numpy(k).to(self.k.dtype)
        self.v[l, b, :, start:start + n] = torch.from_numpy(v).to(self.v.dtype)


# ----------------------------------------------------------------------------- layer math

def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis (no gain)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_cos_sin(positions, head_dim: int, theta: float, prec: Prec):
    """cos/sin of ``pos * theta**(-2j/dh)`` for j < dh/2, angles in float64.

    In bf16 workloads the tables are rounded to binary32, the precision the
    kernels apply them in.
    """
    half = head_dim // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    if prec.bf16:
        c, s = round_fp32(c), round_fp32(s)
    return c, s


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (j, j + dh/2) of ``x[..., n, dh]`` by the angle of row n."""
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal_start: Optional[int] = None):
    """softmax(q k^T / sqrt(dh)) v per head.

    q: [H, n, dh]; k, v: [H, P + n, dh].  With ``causal_start = P`` query i sees
    keys j <= P + i; with None every query sees every key (bidirectional).
    """
    dh = q.shape[-1]
    s = np.einsum("hqd,hkd->hqk", q, k) / math.sqrt(dh)
    if causal_start is not None:
        n, nk = q.shape[1], k.shape[1]
        mask = np.arange(nk)[None, :] > (causal_start + np.arange(n))[:, None]
        s = np.where(mask[None], -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("hqk,hkd->hqd", p, v)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def swiglu(b: np.ndarray, w_gu: np.ndarray, w_d: np.ndarray, prec: Prec) -> np.ndarray:
    """W_down( silu(W_gate b) * (W_up b) ); ``w_gu`` rows hold gate then up."""
    de = w_gu.shape[0] // 2
    gu = b @ w_gu.T
    u = prec.act(silu(gu[:, :de]) * gu[:, de:])
    return u @ w_d.T


def route(r32: np.ndarray, k: int):
    """Top-k experts per row by router logit (ties: lower id) and their weights.

    The weights are the router softmax restricted to the k picks and
    renormalised, i.e. a softmax over the k picked logits.
    """
    T, E = r32.shape
    ids = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-r32[t, e], e))
        ids[t] = order[:k]
    sel = np.take_along_axis(r32, ids, axis=1)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return ids, w


def moe(b: np.ndarray, W: Weights, l: int, prec: Prec, k: int, E: int):
    """Routed experts plus the shared expert, summed in float64.

    With MXFP4 x MXFP8 experts the routed gate/up reads each token row as
    MXFP8 (E4M3 elements, one E8M0 scale per 32 along d_model); the down
    projection and the shared expert read their inputs as they are.
    """
    r32 = round_fp32(b @ W.dense(l, "wr").T)
    ids, w = route(r32, k)
    out = np.zeros_like(b)
    bq = round_mxfp8(b) if W.cfg.expert_dtype == "mxfp4_a8" else b
    for e in range(E):
        rows, slot = np.nonzero(ids == e)
        if rows.size == 0:
            continue
        w_gu, w_d = W.expert(l, e)
        out[rows] += w[rows, slot][:, None] * swiglu(bq[rows], w_gu, w_d, prec)
    out += swiglu(b, W.dense(l, "ws_gu"), W.dense(l, "ws_d"), prec)
    return out, ids, w, r32


def layer_forward(x, W: Weights, l: int, kvk, kvv, P: int, prec: Prec, cfg,
                  causal: bool = False, kv_only: bool = False, trace: Optional[dict] = None):
    """One pre-norm block for the n rows of one canvas at positions P..P+n-1.

    ``kvk``/``kvv``: cached keys/values [H, P, dh] (already rotary-embedded).
    Returns (x_out, k_new, v_new); with ``kv_only`` x_out is None.
    """
    n = x.shape[0]
    H, dh, A = cfg.n_heads, cfg.head_dim, cfg.attn_dim
    a = prec.act(rmsnorm(x, cfg.rms_eps))
    qkv = prec.act(a @ W.dense(l, "wqkv").T)
    q = qkv[:, :A].reshape(n, H, dh).transpose(1, 0, 2)
    k = qkv[:, A:2 * A].reshape(n, H, dh).transpose(1, 0, 2)
    v = qkv[:, 2 * A:].reshape(n, H, dh).transpose(1, 0, 2)
    if cfg.rope_theta > 0:
        cos, sin = rope_cos_sin(np.arange(P, P + n), dh, cfg.rope_theta, prec)
        q = prec.act(apply_rope(q, cos, sin))
        k = prec.act(apply_rope(k, cos, sin))
    if kv_only:
        return None, k, v
    K = np.concatenate([kvk, k], axis=1)
    V = np.concatenate([kvv, v], axis=1)
    o = prec.act(attention(q, K, V, causal_start=P if causal else None))
    o = o.transpose(1, 0, 2).reshape(n, A)
    x = prec.act(x + o @ W.dense(l, "wo").T)
    b = prec.act(rmsnorm(x, cfg.rms_eps))
    m, ids, w, r32 = moe(b, W, l, prec, cfg.top_k, cfg.n_experts)
    x = prec.act(x + m)
    if trace is not None:
        trace.setdefault("route_ids", []).append(ids)
        trace.setdefault("route_r32", []).append(r32)
    return x, k, v


# ----------------------------------------------------------------------------- confidence

def confidence(z: np.ndarray):
    """Per-row entropy (nats), argmax and top-2 gap of logits ``z[n, V]``.

    Entropy is that of softmax(z): H = logsumexp(z) - sum_v softmax(z)_v z_v.
    The argmax (lowest id on ties) and the gap are taken on binary32 logits and
    the entropy is returned rounded to binary32, the precision decisions use.
    """
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    S = e.sum(axis=1)
    H = np.log(S) - (e * (z - m)).sum(axis=1) / S
    z32 = round_fp32(z)
    a = np.argmax(z32, axis=1)
    top2 = np.sort(np.partition(z32, -2, axis=1)[:, -2:], axis=1)
    gap = top2[:, 1] - top2[:, 0]
    return round_fp32(H), a.astype(np.int64), gap


def lm_head_logits(hf: np.ndarray, W: Weights) -> np.ndarray:
    z = np.empty((hf.shape[0], W.cfg.vocab), dtype=np.float64)
    for c0, c1, w in W.lm_head_chunks():
        z[:, c0:c1] = hf @ w.T
    return z


# ----------------------------------------------------------------------------- commit / noise

def _rank_key(H32: float, i: int):
    # NaN entropies rank after every number.
    return (1, 0.0, i) if math.isnan(H32) else (0, H32, i)


def commit_count(U: int, s: int, max_steps: int) -> int:
    """m = ceil(U / (S_max - s)) for 0-based step s < S_max."""
    return -(-U // (max_steps - s)) if U else 0


def commit_select(H32, a, tok, committed, s: int, max_steps: int, threshold: float):
    """Commit the m lowest-(entropy, position) uncommitted positions plus every
    uncommitted one with entropy below ``threshold``; write their argmax.

    Mutates ``tok``/``committed`` (one canvas) and returns the boolean mask of
    positions committed by this step.
    """
    unc = [i for i in range(len(tok)) if not committed[i]]
    m = commit_count(len(unc), s, max_steps)
    ranked = sorted(unc, key=lambda i: _rank_key(float(H32[i]), i))
    chosen = set(ranked[:m])
    chosen |= {i for i in unc if float(H32[i]) < threshold}
    newly = np.zeros(len(tok), dtype=bool)
    for i in chosen:
        tok[i] = a[i]
        committed[i] = True
        newly[i] = True
    return newly


# Noise.  The method's own noise is uniform-state: every uncommitted position
# gets a fresh uniform id.  The masked (absorbing-state) diffusion the pages
# contrast it with (DiffusionGemma深度拆解 (zhichai.net), "统一状态扩散 vs
# 掩码扩散": a token is either known or masked, and denoising reveals it) is
# the variant selected by mask_token >= 0: the canvas starts as all [MASK]
# and an uncommitted position goes back to [MASK] after each step.

def canvas_init(seed: int, n: int, canvas: int, block: int, vocab: int, mask_token: int = -1):
    if mask_token >= 0:
        return np.full(n, mask_token, dtype=np.int64)
    return philox.canvas_draw(seed, np.arange(n), 0, canvas, block, vocab)


def renoise(tok, committed, seed: int, s: int, canvas: int, block: int, vocab: int, mask_token: int = -1):
    """Redraw every uncommitted position uniformly (counter step tag s + 1),
    or set it to [MASK] under absorbing-state noise."""
    idx = np.nonzero(~np.asarray(committed, dtype=bool))[0]
    if idx.size:
        tok[idx] = mask_token if mask_token >= 0 else philox.canvas_draw(seed, idx, s + 1, canvas, block, vocab)


# ----------------------------------------------------------------------------- step / loop

@dataclass
class CanvasState:
    tokens: np.ndarray          # int64 [B, N]
    committed: np.ndarray       # bool  [B, N]
    step: int = 0
    seed: int = 0
    block: int = 0
    prediction: Optional[np.ndarray] = None   # int64 [B, N]: previous step's argmax (self-conditioning)

    def copy(self):
        return CanvasState(self.tokens.copy(), self.committed.copy(), self.step, self.seed,
                           self.block, None if self.prediction is None else self.prediction.copy())


@dataclass
class StepResult:
    entropy: np.ndarray          # float64 (binary32 values) [B, N]
    argmax: np.ndarray           # int64 [B, N]
    gap: np.ndarray              # [B, N]
    newly: np.ndarray            # bool [B, N]
    n_uncommitted: np.ndarray    # int [B] after the commit
    cutoff: np.ndarray           # m-th smallest uncommitted entropy per canvas (nan if m == 0)
    m: np.ndarray                # commit count per canvas
    logits: Optional[np.ndarray] = None
    hidden: Optional[np.ndarray] = None
    trace: dict = field(default_factory=dict)


def init_state(cfg, seed: int, block: int = 0) -> CanvasState:
    B, N = cfg.batch, cfg.canvas_len
    mt = getattr(cfg, "mask_token", -1)
    tok = np.stack([canvas_init(seed, N, b, block, cfg.vocab, mt) for b in range(B)])
    return CanvasState(tok, np.zeros((B, N), dtype=bool), 0, seed, block)


def prefill(state: CanvasState, tokens: np.ndarray, mask: np.ndarray) -> CanvasState:
    """Fix known positions before the first step (fill-in-the-middle, puzzles
    with givens: DiffusionGemma深度拆解 (zhichai.net), "代码填充的结构性优势" --
    bidirectional attention lets the open positions use the known tokens on
    both sides).  Where ``mask`` [B, N] is set the canvas takes ``tokens`` and
    the position counts as committed: it is fed to every forward like any
    committed token, never ranked, counted in U or re-noised.
    """
    if state.step != 0:
        raise ValueError("prefill applies to a canvas before its first step")
    m = np.asarray(mask, dtype=bool)
    state.tokens[m] = np.asarray(tokens, dtype=np.int64)[m]
    state.committed |= m
    return state


def input_embedding(tok_row, W: Weights, prec: Prec, cond_row=None) -> np.ndarray:
    """Input rows of a canvas: the token embeddings, plus (self-conditioning)
    the embeddings of the previous step's predictions, summed before one
    rounding to the activation precision."""
    e = W.embed_rows(tok_row)
    if cond_row is not None:
        e = e + W.embed_rows(cond_row)
    return prec.act(e)


def forward_canvas(tok_row, W: Weights, kv: KV, b: int, cfg, prec: Prec, trace=None, cond_row=None):
    """Bidirectional forward of one canvas; returns the final normed hidden rows.
    ``cond_row``: the previous step's predictions (self-conditioning) or None."""
    P = kv.length
    x = input_embedding(tok_row, W, prec, cond_row)
    for l in range(cfg.n_layers):
        kvk, kvv = kv.get(l, b)
        x, _, _ = layer_forward(x, W, l, kvk, kvv, P, prec, cfg, trace=trace)
    return prec.act(rmsnorm(x, cfg.rms_eps))


def denoise_step(W: Weights, kv: KV, state: CanvasState, cfg, keep_logits: bool = False,
                 keep_hidden: bool = False, hook: Optional[Callable] = None) -> StepResult:
    """One denoise step for every canvas of ``state`` (mutated in place).

    Forward all positions, score them, commit, then re-noise the rest.
    ``hook(result, state)`` (tests) runs after the commit and before re-noise.
    """
    prec = Prec(cfg.act_dtype)
    B, N = state.tokens.shape
    s = state.step
    if s >= cfg.max_steps:
        raise ValueError("step cap reached")
    Hs, As, Gs, NW, Ls, Hid = [], [], [], [], [], []
    Up, cut, ms = np.zeros(B, dtype=np.int64), np.full(B, np.nan), np.zeros(B, dtype=np.int64)
    trace = {}
    cond = getattr(cfg, "self_condition", False) and state.prediction is not None
    for b in range(B):
        hf = forward_canvas(state.tokens[b], W, kv, b, cfg, prec, trace=trace,
                            cond_row=state.prediction[b] if cond else None)
        z = lm_head_logits(hf, W)
        H32, a, gap = confidence(z)
        unc = ~state.committed[b]
        U = int(unc.sum())
        m = commit_count(U, s, cfg.max_steps)
        ms[b] = m
        if m:
            ranked = sorted(np.nonzero(unc)[0], key=lambda i: _rank_key(float(H32[i]), int(i)))
            cut[b] = H32[ranked[m - 1]]
        newly = commit_select(H32, a, state.tokens[b], state.committed[b], s, cfg.max_steps,
                              cfg.threshold)
        Up[b] = int((~state.committed[b]).sum())
        Hs.append(H32); As.append(a); Gs.append(gap); NW.append(newly)
        if keep_logits:
            Ls.append(z)
        if keep_hidden:
            Hid.append(hf)
    res = StepResult(np.stack(Hs), np.stack(As), np.stack(Gs), np.stack(NW), Up, cut, ms,
                     np.stack(Ls) if keep_logits else None,
                     np.stack(Hid) if keep_hidden else None, trace)
    if hook is not None:
        hook(res, state)
    for b in range(B):
        renoise(state.tokens[b], state.committed[b], state.seed, s, b, state.block, cfg.vocab,
                getattr(cfg, "mask_token", -1))
    if getattr(cfg, "self_condition", False):
        state.prediction = res.argmax.copy()
    state.step = s + 1
    return res


def generate_canvas(W: Weights, kv: KV, cfg, seed: int, block: int = 0,
                    state: Optional[CanvasState] = None, hook: Optional[Callable] = None,
                    step_hook: Optional[Callable] = None):
    """Denoise until every canvas is committed or the step cap is reached.

    Returns (state, steps_taken).
    """
    if state is None:
        state = init_state(cfg, seed, block)
    while state.step < cfg.max_steps:
        res = denoise_step(W, kv, state, cfg, hook=hook)
        if step_hook is not None:
            step_hook(res, state)
        if int(res.n_uncommitted.sum()) == 0:
            break
    return state, state.step


def commit_canvas(W: Weights, kv: KV, tokens: np.ndarray, cfg):
    """Causal pass over ``tokens[B, n]`` at positions P..P+n-1 that appends their
    rotary-embedded K and V to every layer's cache; ``kv.length += n``.
    """
    prec = Prec(cfg.act_dtype)
    B, n = tokens.shape
    P = kv.length
    if P + n > kv.capacity:
        raise ValueError("KV capacity exceeded")
    for b in range(B):
        x = prec.act(W.embed_rows(tokens[b]))
        for l in range(cfg.n_layers):
            kvk, kvv = kv.get(l, b, P)
            last = l == cfg.n_layers - 1
            x, k, v = layer_forward(x, W, l, kvk, kvv, P, prec, cfg, causal=True, kv_only=last)
            kv.put(l, b, P, k, v)
    kv.length = P + n


def block_generate(W: Weights, kv: KV, cfg, prompt_tokens: np.ndarray):
    """Encode the prompt, then generate and append ``cfg.n_canvases`` canvases."""
    commit_canvas(W, kv, prompt_tokens, cfg)
    outs, steps = [], []
    for c in range(cfg.n_canvases):
        st, taken = generate_canvas(W, kv, cfg, cfg.seed, block=c)
        commit_canvas(W, kv, st.tokens, cfg)
        outs.append(st.tokens.copy())
        steps.append(taken)
    return outs, steps
