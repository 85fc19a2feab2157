"""Oracle pins for the per-layer math: RMSNorm, RoPE, attention, router, MoE,
and the entropy/argmax confidence.  Each is checked against a library routine
or a closed form, never against a retyped copy of its own formula."""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import model as om
from workloads import make_inputs, tiny_config

RNG = np.random.default_rng(123)


# ----------------------------------------------------------------------------- entropy

def test_entropy_uniform_is_log_v():
    for V in (512, 262144):
        H, a, gap = om.confidence(np.zeros((2, V)))
        np.testing.assert_allclose(H, math.log(V), rtol=0, atol=2e-6)
        assert (a == 0).all() and (gap == 0).all()
    assert abs(math.log(512) - 6.238324625039508) < 1e-15
    assert abs(math.log(262144) - 12.476649250079015) < 1e-15


def test_entropy_one_hot_is_zero_and_k_way_tie_is_log_k():
    z = np.full((3, 64), -1e4)
    z[0, 17] = 0.0
    z[1, [5, 9]] = 3.0
    z[2, [1, 2, 40, 63]] = -2.0
    H, a, gap = om.confidence(z)
    np.testing.assert_allclose(H, [0.0, math.log(2), math.log(4)], atol=1e-7)
    np.testing.assert_array_equal(a, [17, 5, 1])     # lowest index among ties
    np.testing.assert_array_equal(gap[1:], [0.0, 0.0])


def test_entropy_matches_scipy():
    z = RNG.standard_normal((8, 4096)) * np.array([0.1, 1, 3, 6, 10, 20, 50, 100])[:, None]
    H, a, gap = om.confidence(z)
    p = scipy.special.softmax(z, axis=1)
    ref = scipy.stats.entropy(p, axis=1)
    np.testing.assert_allclose(H, ref, rtol=2e-7, atol=2e-6)
    lse = scipy.special.logsumexp(z, axis=1)
    np.testing.assert_allclose(H, lse - (p * z).sum(1), rtol=2e-7, atol=2e-6)
    np.testing.assert_array_equal(a, np.argmax(z.astype(np.float32), axis=1))
    srt = np.sort(z.astype(np.float32), axis=1)
    np.testing.assert_allclose(gap, srt[:, -1].astype(np.float64) - srt[:, -2], rtol=1e-6)


# ----------------------------------------------------------------------------- rmsnorm / rope

def test_rmsnorm_unit_rms_and_torch():
    x = RNG.standard_normal((16, 256)) * 5
    y = om.rmsnorm(x, 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(1)), 1.0, rtol=1e-12)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (256,), eps=1e-6).numpy()
    np.testing.assert_allclose(om.rmsnorm(x, 1e-6), ref, rtol=1e-12)
    np.testing.assert_allclose(om.rmsnorm(7.0 * x, 0.0), y, rtol=1e-12)   # scale invariance


def test_rope_is_complex_rotation():
    prec = om.Prec("fp32")
    dh, n = 16, 40
    x = RNG.standard_normal((3, n, dh))
    pos = np.arange(100, 100 + n)
    c, s = om.rope_cos_sin(pos, dh, 1e4, prec)
    y = om.apply_rope(x, c, s)
    # pair (j, j + dh/2) as the complex number x_j + i x_{j+dh/2}, times e^{i pos theta^(-2j/dh)}
    zc = (x[..., :dh // 2] + 1j * x[..., dh // 2:]) * np.exp(
        1j * pos[:, None] * 1e4 ** (-np.arange(dh // 2) * 2.0 / dh))
    np.testing.assert_allclose(y, np.concatenate([zc.real, zc.imag], -1), atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    c0, s0 = om.rope_cos_sin(np.zeros(1), dh, 1e4, prec)
    np.testing.assert_allclose(om.apply_rope(x[:, :1], c0, s0), x[:, :1], atol=0)


def test_rope_scores_depend_only_on_offset():
    prec = om.Prec("fp32")
    dh = 32
    q, k = RNG.standard_normal(dh), RNG.standard_normal(dh)

    def score(m, n):
        cm, sm = om.rope_cos_sin([m], dh, 1e4, prec)
        cn, sn = om.rope_cos_sin([n], dh, 1e4, prec)
        return float((om.apply_rope(q[None], cm, sm) @ om.apply_rope(k[None], cn, sn).T)[0, 0])
    assert abs(score(10, 3) - score(1007, 1000)) < 1e-9
    assert abs(score(0, 0) - float(q @ k)) < 1e-12


# ----------------------------------------------------------------------------- attention

def _sdpa(q, k, v, mask=None):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None, None]).numpy()[0]


def test_attention_bidirectional_matches_torch_sdpa():
    H, P, n, dh = 3, 11, 7, 16
    q = RNG.standard_normal((H, n, dh))
    k = RNG.standard_normal((H, P + n, dh))
    v = RNG.standard_normal((H, P + n, dh))
    np.testing.assert_allclose(om.attention(q, k, v), _sdpa(q, k, v), rtol=1e-12, atol=1e-12)


def test_attention_causal_matches_torch_sdpa():
    H, P, n, dh = 2, 9, 6, 8
    q = RNG.standard_normal((H, n, dh))
    k = RNG.standard_normal((H, P + n, dh))
    v = RNG.standard_normal((H, P + n, dh))
    allowed = np.arange(P + n)[None, :] <= (P + np.arange(n))[:, None]
    np.testing.assert_allclose(om.attention(q, k, v, causal_start=P), _sdpa(q, k, v, allowed),
                               rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    H, dh = 2, 8
    q = RNG.standard_normal((H, 5, dh))
    v = RNG.standard_normal((H, 9, dh))
    same = np.repeat(RNG.standard_normal((H, 1, dh)), 9, axis=1)
    np.testing.assert_allclose(om.attention(q, same, v), np.repeat(v.mean(1, keepdims=True), 5, 1),
                               atol=1e-12)
    k1, v1 = RNG.standard_normal((H, 1, dh)), RNG.standard_normal((H, 1, dh))
    np.testing.assert_allclose(om.attention(q, k1, v1), np.repeat(v1, 5, 1), atol=1e-12)


def test_attention_permutation_equivariance():
    H, P, n, dh = 2, 13, 10, 8
    q = RNG.standard_normal((H, n, dh))
    kp, vp = RNG.standard_normal((H, P, dh)), RNG.standard_normal((H, P, dh))
    kc, vc = RNG.standard_normal((H, n, dh)), RNG.standard_normal((H, n, dh))
    base = om.attention(q, np.concatenate([kp, kc], 1), np.concatenate([vp, vc], 1))
    pc, pp = RNG.permutation(n), RNG.permutation(P)
    out = om.attention(q[:, pc], np.concatenate([kp[:, pp], kc[:, pc]], 1),
                       np.concatenate([vp[:, pp], vc[:, pc]], 1))
    np.testing.assert_allclose(out, base[:, pc], atol=1e-12)


# ----------------------------------------------------------------------------- router / MoE

def test_route_brute_force_and_ties():
    r = RNG.standard_normal((50, 8)).round(1)           # rounding creates ties
    ids, w = om.route(r, 3)
    for t in range(50):
        best = sorted(range(8), key=lambda e: (-r[t, e], e))[:3]
        assert list(ids[t]) == best
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    ids, w = om.route(np.zeros((4, 8)), 3)
    np.testing.assert_array_equal(ids, [[0, 1, 2]] * 4)
    np.testing.assert_allclose(w, 1.0 / 3)


def test_route_weights_equal_renormalised_softmax():
    r = RNG.standard_normal((20, 16))
    ids, w = om.route(r, 4)
    p = scipy.special.softmax(r, axis=1)
    sel = np.take_along_axis(p, ids, 1)
    np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-12)


def _moe_inputs(**kw):
    cfg = tiny_config(**kw)
    inp = make_inputs(cfg)
    return cfg, inp


def test_moe_single_expert_is_dense_swiglu_via_torch():
    cfg, inp = _moe_inputs(n_experts=1, top_k=1)
    W = om.Weights(inp, cache=True)
    b = RNG.standard_normal((9, cfg.d_model))
    out, ids, w, _ = om.moe(b, W, 0, om.Prec("fp32"), 1, 1)
    assert (ids == 0).all() and np.allclose(w, 1.0)
    tb = torch.from_numpy(b)
    lin = torch.nn.functional.linear

    def dense(gu, dw):
        g, u = lin(tb, torch.from_numpy(gu)).chunk(2, dim=-1)
        return lin(torch.nn.functional.silu(g) * u, torch.from_numpy(dw))
    e_gu, e_d = W.expert(0, 0)
    ref = dense(e_gu, e_d) + dense(W.dense(0, "ws_gu"), W.dense(0, "ws_d"))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_moe_identical_experts_ignore_routing():
    cfg, inp = _moe_inputs()
    for name in ("w_gu", "w_d"):
        inp.layers[0][name][:] = inp.layers[0][name][0:1].clone()
    W = om.Weights(inp, cache=True)
    b = RNG.standard_normal((12, cfg.d_model))
    out, ids, w, _ = om.moe(b, W, 0, om.Prec("fp32"), cfg.top_k, cfg.n_experts)
    e_gu, e_d = W.expert(0, 0)
    ref = om.swiglu(b, e_gu, e_d, om.Prec("fp32")) + om.swiglu(
        b, W.dense(0, "ws_gu"), W.dense(0, "ws_d"), om.Prec("fp32"))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_moe_each_expert_block_is_a_plain_matmul():
    cfg, inp = _moe_inputs()
    W = om.Weights(inp, cache=True)
    b = RNG.standard_normal((30, cfg.d_model))
    out, ids, w, _ = om.moe(b, W, 0, om.Prec("fp32"), cfg.top_k, cfg.n_experts)
    assert np.bincount(ids.ravel(), minlength=cfg.n_experts).sum() == 30 * cfg.top_k
    # rebuild from per-token loops with torch matmuls in a different association order
    ref = np.zeros_like(b)
    for t in range(30):
        for j in range(cfg.top_k):
            gu, dw = (torch.from_numpy(a) for a in W.expert(0, int(ids[t, j])))
            h = gu @ torch.from_numpy(b[t])
            de = h.shape[0] // 2
            ref[t] += w[t, j] * (dw @ (torch.nn.functional.silu(h[:de]) * h[de:])).numpy()
    ref += om.swiglu(b, W.dense(0, "ws_gu"), W.dense(0, "ws_d"), om.Prec("fp32"))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_fp8_expert_dequant_matches_torch():
    cfg = tiny_config(act_dtype="bf16", expert_dtype="fp8")
    inp = make_inputs(cfg)
    W = om.Weights(inp)
    lw = inp.layers[0]
    got, _ = W.expert(0, 3)
    ref = (lw["w_gu"][3].view(torch.float8_e4m3fn).double() * lw["s_gu"][3].double()[:, None])
    np.testing.assert_array_equal(got, ref.numpy())


def test_moe_mxfp8_inputs_reach_only_the_routed_gate_up():
    """MXFP4 x MXFP8 experts: the routed gate/up reads its token rows as MXFP8
    values, nothing else does.  (1) Rows already on the MXFP8 grid give the
    MXFP4 result exactly (the SwiGLU products entering the down projection are
    off the grid, so quantizing them would show); (2) with zero routed
    weights the shared expert alone gives the MXFP4 result on rows off the
    grid; (3) with one expert and a zero shared expert, raw rows give the
    MXFP4 result of the quantized rows, and not of the raw ones."""
    from oracle.numerics import round_mxfp8
    prec = om.Prec("bf16")

    def pair(**kw):
        ws = []
        for edt in ("mxfp4_a8", "mxfp4"):
            inp = make_inputs(tiny_config(act_dtype="bf16", expert_dtype=edt, **kw))
            ws.append(inp)
        return ws

    a8, f4 = pair()
    cfg = a8.cfg
    b = om.round_bf16(RNG.standard_normal((12, cfg.d_model)))
    bq = round_mxfp8(b)
    assert not np.array_equal(bq, b)
    run = lambda inp, x: om.moe(x, om.Weights(inp), 0, prec, cfg.top_k, cfg.n_experts)[0]
    np.testing.assert_array_equal(run(a8, bq), run(f4, bq))
    for inp in (a8, f4):
        inp.layers[0]["w_gu"].zero_()
    np.testing.assert_array_equal(run(a8, b), run(f4, b))
    a8, f4 = pair(n_experts=1, top_k=1)
    for inp in (a8, f4):
        inp.layers[0]["ws_gu"].zero_()
    one = lambda inp, x: om.moe(x, om.Weights(inp), 0, prec, 1, 1)[0]
    np.testing.assert_array_equal(one(a8, b), one(f4, bq))
    assert not np.allclose(one(a8, b), one(f4, b), rtol=1e-6, atol=0)


def test_block_matches_torch_functional_composition():
    """One whole block against an independent composition of torch library ops:
    F.linear fixes the [out][in] weight orientation, SDPA fixes attention, the
    rotary embedding is a complex multiplication, top-k comes from torch.topk."""
    cfg = tiny_config(seed=3)
    inp = make_inputs(cfg)
    W = om.Weights(inp, cache=True)
    kv = om.KV(inp.kv_k, inp.kv_v, inp.kv_len, bf16=False)
    n, P, H, dh, d = cfg.canvas_len, cfg.prompt_len, cfg.n_heads, cfg.head_dim, cfg.d_model
    x = RNG.standard_normal((n, d))
    kvk, kvv = kv.get(0, 0)
    got, k_new, v_new = om.layer_forward(x, W, 0, kvk, kvv, P, om.Prec("fp32"), cfg)

    F = torch.nn.functional
    lw = {k: (v.double() if v is not None else None) for k, v in inp.layers[0].items()}
    tx = torch.from_numpy(x)
    a = F.rms_norm(tx, (d,), eps=cfg.rms_eps)
    q, k, v = F.linear(a, lw["wqkv"]).split(H * dh, dim=-1)
    pos = torch.arange(P, P + n, dtype=torch.float64)
    inv = cfg.rope_theta ** (-torch.arange(dh // 2, dtype=torch.float64) * 2 / dh)
    rot = torch.polar(torch.ones(n, dh // 2, dtype=torch.float64), pos[:, None] * inv[None])

    def rope(t):  # t [n, H, dh]
        c = torch.complex(t[..., :dh // 2], t[..., dh // 2:]) * rot[:, None, :]
        return torch.cat([c.real, c.imag], dim=-1)
    q = rope(q.view(n, H, dh)).transpose(0, 1)
    k = rope(k.view(n, H, dh)).transpose(0, 1)
    v = v.view(n, H, dh).transpose(0, 1)
    K = torch.cat([torch.from_numpy(kvk), k], 1)
    V = torch.cat([torch.from_numpy(kvv), v], 1)
    o = F.scaled_dot_product_attention(q[None], K[None], V[None])[0].transpose(0, 1).reshape(n, -1)
    h = tx + F.linear(o, lw["wo"])
    b = F.rms_norm(h, (d,), eps=cfg.rms_eps)
    logits = F.linear(b, lw["wr"]).float().double()
    top, ids = torch.topk(logits, cfg.top_k, dim=-1)
    wts = torch.softmax(top, dim=-1)

    def swi(inp_, gu, dw):
        g, u = F.linear(inp_, gu).chunk(2, dim=-1)
        return F.linear(F.silu(g) * u, dw)
    moe = torch.zeros_like(b)
    for t in range(n):
        for j in range(cfg.top_k):
            e = int(ids[t, j])
            moe[t] += wts[t, j] * swi(b[t], lw["w_gu"][e], lw["w_d"][e])
    ref = h + moe + swi(b, lw["ws_gu"], lw["ws_d"])
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(k_new, k.numpy(), rtol=1e-12, atol=1e-12)
