"""Oracle-side references and error bounds for the kernel unit tests (test
infrastructure; imports the oracle).

A kernel that rounds to bfloat16 is checked element by element against the
oracle's float64 value: each element must be the oracle's rounding, except
where the oracle's unrounded value lies within the kernel's stated fp32 error
bound of a bf16 rounding boundary -- there either neighbour is correct.  The
bounds follow the arithmetic, not a measurement:

* a dot product over K accumulated by 16x16x32 bf16 MFMA steps in fp32 (exact
  bf16 products) takes at most K/32 accumulator roundings, each at most
  2^-24 of the partial sum, so |error| <= (K/32) 2^-24 sum|a_k w_k|, plus one
  rounding of the result (2^-24 |result|) for a scale or epilogue product;
* SwiGLU h = silu(g) u from such g and u: |dh| <= 1.1 |u| dg + |silu(g)| du
  (|silu'| <= 1.1) plus 2^-19 |h| for the fp32 exp, division and product;
* attention: each probability carries a relative error below
  eps_q = 2^-21 max_j(sum_d|q_d k_jd|) / sqrt(dh) (score accumulation, in
  nats) + 2^-17 (its two-part bf16 split, 2^-18, and the fp32 exp2 and
  fused scale), and the P.V accumulation at most (keys/16) roundings of
  2^-24; the output moves by at most (eps_q + keys 2^-28) (A(|v|) + |o|),
  A(|v|) the attention-weighted mean of |v|.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import model as om
from oracle.numerics import round_bf16

U24 = 2.0 ** -24


def gemm_tol(a: np.ndarray, w: np.ndarray, out: np.ndarray) -> np.ndarray:
    """Bound on |fp32 MFMA result - exact| for out = a @ w.T (K = a.shape[1])."""
    K = a.shape[-1]
    return (K / 32.0) * U24 * (np.abs(a) @ np.abs(w).T) + U24 * np.abs(out)


def check_bf16(got: np.ndarray, pre: np.ndarray, tol: np.ndarray, what: str, max_frac: float = 5e-3,
               mask=None):
    """Every element of ``got`` (bf16 values as float64) is round_bf16(pre) or,
    where pre lies within tol of a rounding boundary, a value between the
    roundings of pre - tol and pre + tol.  ``mask`` (optional) selects the
    elements checked.  Returns (mismatches, flagged)."""
    got = np.asarray(got, dtype=np.float64)
    pre = np.asarray(pre, dtype=np.float64)
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), pre.shape)
    if mask is not None:
        got, pre, tol = got[mask], pre[mask], tol[mask]
    exp = round_bf16(pre)
    lo, hi = round_bf16(pre - tol), round_bf16(pre + tol)
    flagged = lo != hi
    exact = got == exp
    ok = exact | (flagged & (got >= lo) & (got <= hi))
    bad = np.argwhere(~ok)
    assert bad.size == 0, (f"{what}: {len(bad)} elements off by more than the bound, first at "
                           f"{tuple(bad[0])}: got {got[tuple(bad[0])]!r}, oracle {pre[tuple(bad[0])]!r} "
                           f"(bound {tol[tuple(bad[0])]:.3e})")
    nmis = int((~exact).sum())
    assert nmis <= max_frac * got.size, f"{what}: {nmis} of {got.size} elements differ (all within the bound)"
    return nmis, int(flagged.sum())


def check_f32(got: np.ndarray, ref: np.ndarray, tol: np.ndarray, what: str) -> float:
    """|got - ref| <= tol everywhere; returns the largest |got - ref| / tol."""
    d = np.abs(np.asarray(got, dtype=np.float64) - ref)
    r = d / np.maximum(tol, 1e-300)
    w = np.unravel_index(np.argmax(r), r.shape)
    assert r[w] <= 1.0, f"{what}: |diff| {d[w]:.3e} beyond the bound {tol[w]:.3e} at {w}"
    return float(r[w])


# ----------------------------------------------------------------------------- phases

def qkv_rope_ref(a: np.ndarray, wqkv: np.ndarray, B: int, n: int, H: int, dh: int, pos0: int, theta: float):
    """Oracle q, k, v [B, H, n, dh] (bf16 values) of a [B*n, d], with the bounds:
    returns dict name -> (pre-rounding value, bound, checkable mask)."""
    A = H * dh
    pre = a @ wqkv.T
    tol = gemm_tol(a, wqkv, pre)
    x = round_bf16(pre)
    amb = round_bf16(pre - tol) != round_bf16(pre + tol)

    def heads(t):  # [B*n, A] -> [B, H, n, dh]
        return t.reshape(B, n, H, dh).transpose(0, 2, 1, 3)
    out = {}
    cos, sin = om.rope_cos_sin(np.arange(pos0, pos0 + n), dh, theta, om.Prec("bf16"))
    half = dh // 2
    for name, sl in (("q", slice(0, A)), ("k", slice(A, 2 * A))):
        xv, av = heads(x[:, sl]), heads(amb[:, sl])
        rot = om.apply_rope(xv, cos, sin)
        x1, x2 = xv[..., :half], xv[..., half:]
        mag = np.concatenate([np.abs(x1 * cos) + np.abs(x2 * sin), np.abs(x2 * cos) + np.abs(x1 * sin)], -1)
        # the partner of a rotate-half pair enters every output of the pair
        pair_amb = av[..., :half] | av[..., half:]
        checkable = ~np.concatenate([pair_amb, pair_amb], -1)
        out[name] = (rot, 2.0 ** -22 * mag, checkable)
    out["v"] = (heads(pre[:, 2 * A:]), heads(tol[:, 2 * A:]), np.ones((B, H, n, dh), dtype=bool))
    return out


def attention_ref(q: np.ndarray, K: np.ndarray, V: np.ndarray, causal_start=None):
    """Oracle output (unrounded) of one (canvas, head) and its bound.
    q [n, dh]; K, V [keys, dh]."""
    dh = q.shape[-1]
    o = om.attention(q[None], K[None], V[None], causal_start=causal_start)[0]
    av = om.attention(q[None], K[None], np.abs(V)[None], causal_start=causal_start)[0]
    sabs = (np.abs(q) @ np.abs(K).T).max(axis=1, keepdims=True)
    eps = 2.0 ** -21 * sabs / math.sqrt(dh) + 2.0 ** -17
    keys = K.shape[0]
    tol = (eps + keys * 2.0 ** -28) * (av + np.abs(o))
    return o, tol


def scaled_mfma_tol(a: np.ndarray, w: np.ndarray, out: np.ndarray) -> np.ndarray:
    """Bound on |result - exact| for out = a @ w.T on gfx950's scaled MFMA
    (4-bit x 8-bit operands, 128 k per instruction, fp32 accumulator).  Its
    internal summation is not exact: on random E2M1 x E4M3 operands with
    block scales over 2^-7 .. 2^7 one instruction came within 2^-13.3 of the
    sum of |products| (measured on the device; no published figure is at
    hand).  Over K = 2048 (16 instructions into one accumulator) the bound
    taken is 2^-11 of sum |a_k w_k|, plus one rounding of the result."""
    return 2.0 ** -11 * (np.abs(a) @ np.abs(w).T) + U24 * np.abs(out)


def swiglu_ref(x: np.ndarray, w_gu: np.ndarray, scaled_mfma: bool = False):
    """h = silu(g) u (unrounded) of rows x against gate rows then up rows of
    w_gu, and its bound (scaled_mfma: the products ran on the scaled MFMA)."""
    de = w_gu.shape[0] // 2
    gu = x @ w_gu.T
    tgu = (scaled_mfma_tol if scaled_mfma else gemm_tol)(x, w_gu, gu)
    g, u = gu[:, :de], gu[:, de:]
    sg = om.silu(g)
    h = sg * u
    tol = 1.1 * np.abs(u) * tgu[:, :de] + np.abs(sg) * tgu[:, de:] + 2.0 ** -19 * np.abs(h)
    return h, tol
