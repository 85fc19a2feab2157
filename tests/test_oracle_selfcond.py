"""Pins of the oracle's self-conditioning option (every step after the first
adds the embedding row of the previous step's argmax to each position's input).

The reading is pinned against what it fixes independently of the oracle's
own code: a model with no blocks is the final RMSNorm and the LM head, so its
logits have a closed form, computed here with torch's rms_norm in float64;
step 0 has no earlier prediction and equals the step without the option; the
bf16 input row is one rounding of the exact sum (torch's own cast).
"""
import numpy as np
import torch

from oracle import model as om
from workloads import make_inputs, tiny_config

F = torch.nn.functional


def _cfg(**kw):
    args = dict(name="tiny_selfcond", n_layers=0, canvas_len=24, vocab=512, max_steps=6, seed=41,
                self_condition=True)
    args.update(kw)
    return tiny_config(**args)


def _closed_form_logits(inp, cfg, tok, pred):
    """Logits of a model with no blocks: LM head of rms_norm(E[tok] + E[pred])."""
    E = inp.embed.to(torch.float64)
    x = E[torch.from_numpy(tok)] + (E[torch.from_numpy(pred)] if pred is not None else 0)
    h = F.rms_norm(x, (cfg.d_model,), eps=cfg.rms_eps)
    return (h @ inp.lm_head.to(torch.float64).T).numpy()


def test_zero_layer_step_logits_match_the_closed_form():
    cfg = _cfg()
    inp = make_inputs(cfg)
    W = om.Weights(inp)
    kv = om.KV(inp.kv_k, inp.kv_v, inp.kv_len, bf16=False)
    st = om.init_state(cfg, cfg.seed)
    preds = [None]
    for s in range(3):
        tok = st.tokens[0].copy()
        res = om.denoise_step(W, kv, st, cfg, keep_logits=True)
        ref = _closed_form_logits(inp, cfg, tok, preds[-1])
        np.testing.assert_allclose(res.logits[0], ref, rtol=0, atol=1e-12)
        if s:  # the previous prediction changes what the step sees
            assert np.abs(res.logits[0] - _closed_form_logits(inp, cfg, tok, None)).max() > 1e-3
        np.testing.assert_array_equal(st.prediction[0], res.argmax[0])
        preds.append(st.prediction[0].copy())


def test_first_step_equals_the_unconditioned_step():
    cfg = _cfg(n_layers=1, name="tiny_selfcond_1l")
    inp = make_inputs(cfg)
    W = om.Weights(inp, cache=True)
    outs = []
    for sc in (True, False):
        c = cfg.replace(self_condition=sc)
        kv = om.KV(inp.kv_k, inp.kv_v, inp.kv_len, bf16=False)
        st = om.init_state(c, c.seed)
        r0 = om.denoise_step(W, kv, st, c, keep_logits=True)
        r1 = om.denoise_step(W, kv, st, c, keep_logits=True)
        outs.append((r0, r1, st))
    (a0, a1, sa), (b0, b1, sb) = outs
    np.testing.assert_array_equal(a0.logits, b0.logits)
    np.testing.assert_array_equal(a0.argmax, b0.argmax)
    assert sb.prediction is None and sa.prediction is not None
    # from the second step on the two differ
    assert np.abs(a1.logits - b1.logits).max() > 1e-3


def test_bf16_input_row_is_one_rounding_of_the_sum():
    cfg = _cfg(act_dtype="bf16", expert_dtype="bf16", lm_scale=1.0, name="tiny_selfcond_bf16")
    inp = make_inputs(cfg)
    W = om.Weights(inp)
    rng = np.random.default_rng(3)
    tok = rng.integers(0, cfg.vocab, 64)
    pred = rng.integers(0, cfg.vocab, 64)
    got = om.input_embedding(tok, W, om.Prec("bf16"), pred)
    E = inp.embed.to(torch.float64)
    want = (E[torch.from_numpy(tok)] + E[torch.from_numpy(pred)]).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, want)
    # and without a prediction the row is the embedding itself
    np.testing.assert_array_equal(om.input_embedding(tok, W, om.Prec("bf16")), E[torch.from_numpy(tok)].numpy())
