"""Shared driver for the GPU parity tests: run the HIP path and the oracle
step-locked on the same canvas, compare each step, then resynchronise the GPU
canvas to the oracle's state (test infrastructure; imports the oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import model as om
from tests.parity import compare_step, forced_routing, to_host
from workloads import make_inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Pair:
    """The GPU model + KV cache and the oracle weights + KV over one input set."""

    def __init__(self, rt, cfg, kv_len=None, kv_capacity=None, cache=True):
        self.rt, self.cfg = rt, cfg
        self.inp = make_inputs(cfg, device="cuda", kv_capacity=kv_capacity)
        self.model = rt.Model(self.inp)
        n = self.inp.kv_len if kv_len is None else kv_len
        self.kv = rt.KVCache(self.inp.kv_k.clone(), self.inp.kv_v.clone(), n)
        # cache=False converts each weight when used (a 30-layer model in float64 would
        # take ~135 GB of host memory)
        self.W = om.Weights(self.inp, cache=cache)
        self.okv = om.KV(self.inp.kv_k, self.inp.kv_v, n, bf16=cfg.act_dtype == "bf16")

    def close(self):
        self.model.close()

    def kv_rel(self):
        """rel-L2 of the GPU cache rows in use against the oracle's."""
        n = self.kv.length
        out = []
        for g, o in ((self.kv.k, self.okv.k), (self.kv.v, self.okv.v)):
            gg = g[:, :, :, :n].double().cpu().numpy()
            oo = o[:, :, :, :n].double().numpy()
            out.append(float(np.linalg.norm(gg - oo) / max(np.linalg.norm(oo), 1e-30)))
        return out

    def resync_kv(self):
        self.kv.k.copy_(self.okv.k.to(self.kv.k.dtype).to("cuda"))
        self.kv.v.copy_(self.okv.v.to(self.kv.v.dtype).to("cuda"))
        self.kv.length = self.okv.length

    def commit(self, tokens: np.ndarray):
        """Causal commit pass of tokens [B, n] on both sides."""
        t = torch.from_numpy(np.ascontiguousarray(tokens.astype(np.int32))).to("cuda")
        self.rt.commit_canvas(self.model, t, self.kv)
        torch.cuda.synchronize()
        om.commit_canvas(self.W, self.okv, tokens.astype(np.int64), self.cfg)

    def run_locked(self, block=0, max_steps=None, keep_logits=True, prefill=None):
        """Step-locked denoise loop; returns (step reports, oracle final state).
        prefill: optional (tokens [B, N], mask [B, N]) of pre-committed positions.
        Each step runs the oracle first, so that rows whose router logits
        nearly tie can take the oracle's expert picks on the GPU."""
        rt, cfg = self.rt, self.cfg
        ost = om.init_state(cfg, cfg.seed, block)
        B, N = cfg.batch, cfg.canvas_len
        canvas = rt.Canvas.empty(B, N, cfg.seed, block)
        rt.canvas_init(self.model, canvas)
        if prefill is not None:
            ptok, pmask = prefill
            om.prefill(ost, ptok, pmask)
            rt.canvas_prefill(self.model, canvas, torch.from_numpy(ptok.astype(np.int32)).to("cuda"),
                              torch.from_numpy(pmask.astype(np.uint8)).to("cuda"))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(canvas.tokens), ost.tokens)
        np.testing.assert_array_equal(to_host(canvas.committed).astype(bool), ost.committed)
        ent = torch.empty(B, N, dtype=torch.float32, device="cuda")
        am = torch.empty(B, N, dtype=torch.int32, device="cuda")
        gap = torch.empty(B, N, dtype=torch.float32, device="cuda")
        nunc = torch.empty(B, dtype=torch.int32, device="cuda")
        status = torch.empty(1, dtype=torch.int32, device="cuda")
        act = torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32
        hidden = torch.empty(B * N, cfg.d_model, dtype=act, device="cuda")
        logits = torch.empty(B * N, cfg.vocab, dtype=torch.float32, device="cuda") if keep_logits else None
        reps = []
        try:
            for s in range(max_steps or cfg.max_steps):
                say(f"  {cfg.name}: block {block} step {s}")
                pre = ost.copy()
                ores = om.denoise_step(self.W, self.okv, ost, cfg, keep_logits=keep_logits, keep_hidden=True)
                forced, n_forced = forced_routing(ores.trace, cfg, B, N, self.model.max_batch * N)
                rt.test_force_routing(self.model, torch.from_numpy(forced).to("cuda"))
                rt.denoise_step(self.model, canvas, self.kv, entropy=ent, argmax=am, top2_gap=gap,
                                n_uncommitted=nunc, logits=logits, hidden=hidden, status=status)
                torch.cuda.synchronize()
                assert int(to_host(status)[0]) == 0, f"step status {int(to_host(status)[0])}"
                gpu = dict(entropy=to_host(ent), argmax=to_host(am), tokens=to_host(canvas.tokens),
                           committed=to_host(canvas.committed), hidden=to_host(hidden.float()),
                           logits=to_host(logits) if keep_logits else None)
                self.last_ores = ores
                rep = compare_step(cfg, ores, pre, ost, gpu, W=self.W)
                rep.forced_rows = n_forced
                say("   ", rep)
                reps.append(rep)
                assert canvas.step == ost.step
                if getattr(cfg, "self_condition", False):
                    # the step kept its own argmax for the next step's input
                    np.testing.assert_array_equal(to_host(canvas.prediction), gpu["argmax"])
                    canvas.prediction.copy_(torch.from_numpy(ost.prediction.astype(np.int32)))
                canvas.tokens.copy_(torch.from_numpy(ost.tokens.astype(np.int32)))
                canvas.committed.copy_(torch.from_numpy(ost.committed.astype(np.uint8)))
                if int(ores.n_uncommitted.sum()) == 0:
                    break
        finally:
            rt.test_force_routing(self.model, None)
        return reps, ost


def oracle_perturbed_hidden(W, okv, cfg, tokens, trace, frac=0.01, seed=0, eps=None):
    """The oracle's final normed hidden rows [N, d] of canvas ``tokens`` (batch
    1, cache ``okv``) with a random ``frac`` of block 0's outputs moved to the
    neighbouring bf16 value: how far one block's worth of bf16 rounding noise
    carries by the last layer, in the oracle itself.  Rows whose router
    logits nearly tie in some layer of the unperturbed run (``trace``) keep
    that run's expert picks, as the GPU is made to."""
    from oracle.numerics import round_bf16
    from tests.parity import route_eps
    prec = om.Prec(cfg.act_dtype)
    k = cfg.top_k
    eps = route_eps(cfg) if eps is None else eps
    rng = np.random.default_rng(seed)
    plain_route = om.route
    x = prec.act(W.embed_rows(tokens))
    try:
        for l in range(cfg.n_layers):
            r_ref, ids_ref = trace["route_r32"][l], trace["route_ids"][l]
            srt = -np.sort(-r_ref, axis=1)
            near = (srt[:, k - 1] - srt[:, k]) < eps

            def held(r32, kk, near=near, ids_ref=ids_ref):
                ids, _ = plain_route(r32, kk)
                ids[near] = ids_ref[near]
                sel = np.take_along_axis(r32, ids, axis=1)
                w = np.exp(sel - sel.max(axis=1, keepdims=True))
                return ids, w / w.sum(axis=1, keepdims=True)
            om.route = held
            kvk, kvv = okv.get(l, 0)
            x, _, _ = om.layer_forward(x, W, l, kvk, kvv, okv.length, prec, cfg)
            om.route = plain_route
            if l == 0:
                sel = rng.random(x.shape) < frac
                ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x[sel]), 1e-30))) - 7)
                x[sel] = round_bf16(x[sel] + np.where(rng.random(sel.sum()) < 0.5, -ulp, ulp))
    finally:
        om.route = plain_route
    return prec.act(om.rmsnorm(x, cfg.rms_eps))
