"""Pins of the oracle's bfloat16 arithmetic: where the bf16 workloads round.

The bf16 workloads round to bfloat16 at fixed points of the block (embedding
row, RMSNorm outputs, q/k/v before and after RoPE, attention output, each
residual add, the SwiGLU product of every expert) and keep the expert and
shared-expert outputs unrounded until the residual add.  Here the oracle's
forward of a canvas is compared element by element with an independent
composition of torch library ops in float64 that casts to ``torch.bfloat16``
at exactly those points.  Then mistakes are planted in the oracle (on the CPU)
and must each break the agreement: every single rounding left out, and an
extra rounding of the expert outputs or of the summed MoE output.
"""
import numpy as np
import pytest
import torch

from oracle import model as om
from oracle.numerics import round_bf16
from workloads import make_inputs, tiny_config

F = torch.nn.functional


def _cfg():
    # two layers so the hand-over between blocks is covered; 32-dim heads
    return tiny_config(name="tiny_bf16_pin", act_dtype="bf16", expert_dtype="bf16", n_layers=2,
                       n_heads=2, head_dim=32, lm_scale=1.0, seed=17)


def _r(t: torch.Tensor) -> torch.Tensor:
    """torch's own cast to bfloat16 (round to nearest even), back to float64."""
    return t.to(torch.bfloat16).to(torch.float64)


def torch_forward(inp, cfg, tok, P):
    """The final normed hidden rows of one canvas (canvas 0 of the inputs' KV
    cache), composed of torch library ops in float64 with bf16 casts at the
    stated points.  RoPE is a complex multiplication whose cos/sin are taken
    in float64 and cast to binary32 (the precision the kernels apply them
    in); attention is torch's SDPA; the router top-k is torch.topk on binary32
    logits, weighted by a softmax over the picks."""
    d, H, dh, n = cfg.d_model, cfg.n_heads, cfg.head_dim, len(tok)
    A = H * dh
    x = _r(inp.embed.index_select(0, torch.as_tensor(tok, dtype=torch.int64)).double())
    pos = torch.arange(P, P + n, dtype=torch.float64)
    inv = cfg.rope_theta ** (-torch.arange(dh // 2, dtype=torch.float64) * 2 / dh)
    ang = pos[:, None] * inv[None]
    rot = torch.complex(torch.cos(ang).float().double(), torch.sin(ang).float().double())

    def rope(t):  # t [n, H, dh]
        c = torch.complex(t[..., :dh // 2], t[..., dh // 2:]) * rot[:, None, :]
        return torch.cat([c.real, c.imag], dim=-1)

    for l in range(cfg.n_layers):
        lw = {k: v.double() for k, v in inp.layers[l].items() if v is not None}
        a = _r(F.rms_norm(x, (d,), eps=cfg.rms_eps))
        q, k, v = _r(F.linear(a, lw["wqkv"])).split(A, dim=-1)
        q = _r(rope(q.reshape(n, H, dh))).transpose(0, 1)
        k = _r(rope(k.reshape(n, H, dh))).transpose(0, 1)
        v = v.reshape(n, H, dh).transpose(0, 1)
        K = torch.cat([inp.kv_k[l, 0, :, :P].double(), k], 1)
        V = torch.cat([inp.kv_v[l, 0, :, :P].double(), v], 1)
        o = _r(F.scaled_dot_product_attention(q[None], K[None], V[None])[0].transpose(0, 1).reshape(n, A))
        h = _r(x + F.linear(o, lw["wo"]))
        b = _r(F.rms_norm(h, (d,), eps=cfg.rms_eps))
        top, ids = torch.topk(F.linear(b, lw["wr"]).float(), cfg.top_k, dim=-1)
        wts = torch.softmax(top.double(), dim=-1)

        def swi(rows, gu, dw):
            g, u = F.linear(rows, gu).chunk(2, dim=-1)
            return F.linear(_r(F.silu(g) * u), dw)   # expert output: not rounded
        moe = torch.zeros_like(b)
        for t in range(n):
            for j in range(cfg.top_k):
                e = int(ids[t, j])
                moe[t] += wts[t, j] * swi(b[t:t + 1], lw["w_gu"][e], lw["w_d"][e])[0]
        x = _r(h + (moe + swi(b, lw["ws_gu"], lw["ws_d"])))
    return _r(F.rms_norm(x, (d,), eps=cfg.rms_eps)).numpy()


@pytest.fixture(scope="module")
def setup():
    cfg = _cfg()
    inp = make_inputs(cfg)
    tok = om.init_state(cfg, cfg.seed).tokens[0]
    ref = torch_forward(inp, cfg, tok, cfg.prompt_len)
    return cfg, inp, tok, ref


def _oracle_hidden(cfg, inp, tok):
    W = om.Weights(inp, cache=True)
    kv = om.KV(inp.kv_k, inp.kv_v, inp.kv_len, bf16=True)
    return om.forward_canvas(tok, W, kv, 0, cfg, om.Prec("bf16"))


def test_bf16_forward_matches_torch_composition(setup):
    cfg, inp, tok, ref = setup
    got = _oracle_hidden(cfg, inp, tok)
    # both sides end in a bf16 rounding: equal values, element by element
    np.testing.assert_array_equal(got, ref)
    assert np.array_equal(round_bf16(got), got)


def test_every_rounding_point_is_needed(setup, monkeypatch):
    """Leaving out any one of the oracle's roundings changes its result; the
    only rounding whose input is already bf16 (the embedding row: the table is
    stored in bf16) is a no-op by construction."""
    cfg, inp, tok, ref = setup
    orig = om.Prec.act
    state = {"n": 0, "skip": -1, "noop": []}

    def act(self, x):
        i = state["n"]
        state["n"] += 1
        if self.bf16 and np.array_equal(round_bf16(x), np.asarray(x)):
            state["noop"].append(i)
        return x if i == state["skip"] else orig(self, x)

    monkeypatch.setattr(om.Prec, "act", act)
    np.testing.assert_array_equal(_oracle_hidden(cfg, inp, tok), ref)
    calls, noop = state["n"], list(state["noop"])
    assert noop == [0], noop          # call 0 rounds the embedding row
    # per layer: norm, qkv, q RoPE, k RoPE, attention, residual, norm, one SwiGLU
    # product per expert that got tokens, the shared SwiGLU product, residual;
    # then the final norm
    assert calls >= 1 + cfg.n_layers * 10 + 1
    missed = []
    for skip in range(1, calls):
        state.update(n=0, skip=skip, noop=[])
        got = _oracle_hidden(cfg, inp, tok)
        if np.array_equal(got, ref):
            missed.append(skip)
    assert not missed, f"leaving out rounding call(s) {missed} went unnoticed"


def test_extra_rounding_of_expert_outputs_is_noticed(setup, monkeypatch):
    cfg, inp, tok, ref = setup
    orig = om.swiglu
    monkeypatch.setattr(om, "swiglu", lambda b, gu, dw, prec: round_bf16(orig(b, gu, dw, prec)))
    assert not np.array_equal(_oracle_hidden(cfg, inp, tok), ref)


def test_extra_rounding_of_the_moe_sum_is_noticed(setup, monkeypatch):
    cfg, inp, tok, ref = setup
    orig = om.moe

    def moe(*a, **k):
        out, ids, w, r32 = orig(*a, **k)
        return round_bf16(out), ids, w, r32
    monkeypatch.setattr(om, "moe", moe)
    assert not np.array_equal(_oracle_hidden(cfg, inp, tok), ref)


def test_embedding_gather_runs_on_the_host(setup):
    cfg, inp, tok, _ = setup
    W = om.Weights(inp)
    rows = W.embed_rows(tok[:5])
    assert W.embed_table().device.type == "cpu"
    np.testing.assert_array_equal(rows, inp.embed[torch.as_tensor(tok[:5])].double().numpy())
