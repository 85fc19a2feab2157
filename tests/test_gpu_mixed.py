"""GPU parity of mixed-phase batches: requests in different phases -- causal
prompt reads and block commits next to bidirectional canvas refinements --
in one pass of dg_mixed_step, each request checked against the oracle run on
that request alone (its own denoise step or causal pass).

Refine segments go through the step-locked comparison of tests/parity.py
(backbone, decisions from the GPU's own hidden rows at the stated windows,
decisions against the oracle's forward); append segments compare the cache
rows they write.  Integer results (commit masks, canvases, counts, lengths)
are compared bit for bit outside the flagged cases.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import model as om
from tests.parity import assert_reports, compare_step, forced_routing, to_host
from workloads import make_inputs, tiny_config

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def rt():
    from diffusion_decoding_amd import runtime
    runtime._lib.load()
    return runtime


def _free():
    import gc
    gc.collect()
    torch.cuda.empty_cache()


class Request:
    """One request: its batch-1 GPU cache, the oracle's copy, and (refine
    requests) the GPU canvas and the oracle's canvas state."""

    def __init__(self, mix, b, length, seed=None, block=0):
        rt, inp, cfg1 = mix.rt, mix.inp, mix.cfg1
        self.kv = rt.KVCache(inp.kv_k[:, b:b + 1].clone(), inp.kv_v[:, b:b + 1].clone(), length)
        self.okv = om.KV(inp.kv_k[:, b:b + 1], inp.kv_v[:, b:b + 1], length, bf16=cfg1.act_dtype == "bf16")
        self.canvas = self.ost = None
        if seed is not None:
            N = cfg1.canvas_len
            self.canvas = rt.Canvas.empty(1, N, seed, block)
            rt.canvas_init(mix.model, self.canvas)
            self.ost = om.init_state(cfg1, seed, block)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(to_host(self.canvas.tokens), self.ost.tokens)

    def rows_rel(self, r0, r1):
        """rel-L2 of GPU cache rows [r0, r1) against the oracle's (k, v)."""
        out = []
        for g, o in ((self.kv.k, self.okv.k), (self.kv.v, self.okv.v)):
            gg = g[:, :, :, r0:r1].double().cpu().numpy()
            oo = o[:, :, :, r0:r1].double().numpy()
            out.append(float(np.linalg.norm(gg - oo) / max(np.linalg.norm(oo), 1e-30)))
        return out

    def resync(self):
        self.kv.k.copy_(self.okv.k.to(self.kv.k.dtype).to("cuda"))
        self.kv.v.copy_(self.okv.v.to(self.kv.v.dtype).to("cuda"))
        if self.ost is not None:
            self.canvas.tokens.copy_(torch.from_numpy(self.ost.tokens.astype(np.int32)))
            self.canvas.committed.copy_(torch.from_numpy(self.ost.committed.astype(np.uint8)))
            if self.ost.prediction is not None:
                self.canvas.prediction.copy_(torch.from_numpy(self.ost.prediction.astype(np.int32)))


class Mix:
    """A model over ``n_req`` synthetic caches (make_inputs with batch n_req)."""

    def __init__(self, rt, cfg, max_batch, max_tokens, kv_capacity):
        self.rt, self.cfg = rt, cfg
        self.cfg1 = cfg.replace(batch=1)
        self.inp = make_inputs(cfg, device="cuda", kv_capacity=kv_capacity)
        self.model = rt.Model(self.inp, max_batch=max_batch, max_tokens=max_tokens, max_kv=kv_capacity)
        self.W = om.Weights(self.inp, cache=True)

    def close(self):
        self.model.close()

    def run_pass(self, plan, rel_tol):
        """plan: list of (request, tokens or None); None = refine.  Runs the
        oracle per request, then one mixed pass on the GPU, and compares.
        Returns the refine step reports."""
        rt, cfg1, W = self.rt, self.cfg1, self.W
        N, d = cfg1.canvas_len, cfg1.d_model
        k, L = cfg1.top_k, cfg1.n_layers
        rows_alloc = self.model.max_batch * N
        forced = np.full((L, rows_alloc, k), -1, dtype=np.int32)
        act = torch.bfloat16 if cfg1.act_dtype == "bf16" else torch.float32
        segs, checks = [], []
        j = 0
        for req, tok in plan:
            if tok is None:
                pre = req.ost.copy()
                ores = om.denoise_step(W, req.okv, req.ost, cfg1, keep_logits=False, keep_hidden=True)
                f, _ = forced_routing(ores.trace, cfg1, 1, N, N)
                forced[:, j * N:(j + 1) * N] = f   # refine rows are stacked first, in plan order
                j += 1
                out = dict(entropy=torch.empty(N, device="cuda"),
                           argmax=torch.empty(N, dtype=torch.int32, device="cuda"),
                           n_uncommitted=torch.empty(1, dtype=torch.int32, device="cuda"),
                           hidden=torch.empty(N, d, dtype=act, device="cuda"))
                segs.append(rt.Refine(req.kv, req.canvas, **out))
                checks.append(("refine", req, (pre, ores, out)))
            else:
                P0 = req.okv.length
                om.commit_canvas(W, req.okv, tok[None].astype(np.int64), cfg1)
                segs.append(rt.Append(req.kv, torch.from_numpy(tok.astype(np.int32)).to("cuda")))
                checks.append(("append", req, (P0, len(tok))))
        before = {id(req): (req.kv.k.clone(), req.kv.v.clone()) for kind, req, _ in checks if kind == "refine"}
        status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        rt.test_force_routing(self.model, torch.from_numpy(forced).to("cuda"))
        try:
            rt.mixed_step(self.model, segs, status=status)
            torch.cuda.synchronize()
        finally:
            rt.test_force_routing(self.model, None)
        assert int(to_host(status)[0]) == 0, f"status {int(to_host(status)[0])}"
        reps = []
        for kind, req, info in checks:
            if kind == "refine":
                pre, ores, out = info
                gpu = dict(entropy=to_host(out["entropy"])[None], argmax=to_host(out["argmax"])[None],
                           tokens=to_host(req.canvas.tokens), committed=to_host(req.canvas.committed),
                           hidden=to_host(out["hidden"].float()))
                rep = compare_step(cfg1, ores, pre, req.ost, gpu, W=W)
                say("    refine", rep)
                reps.append(rep)
                assert req.canvas.step == req.ost.step
                assert int(to_host(out["n_uncommitted"])[0]) == int((gpu["committed"] == 0).sum())
                if cfg1.self_condition:
                    np.testing.assert_array_equal(to_host(req.canvas.prediction), gpu["argmax"])
                k0, v0 = before[id(req)]
                assert torch.equal(req.kv.k, k0) and torch.equal(req.kv.v, v0), "a refine pass wrote its cache"
                assert req.kv.length == req.okv.length
            else:
                P0, n = info
                assert req.kv.length == req.okv.length == P0 + n
                rel = req.rows_rel(P0, P0 + n)
                say(f"    append rows [{P0}, {P0 + n}): k, v rel-L2 {rel[0]:.2e} {rel[1]:.2e}")
                assert max(rel) <= rel_tol
        for _, req, _ in checks:
            req.resync()
        return reps


def _tiny_mix(rt, act, **kw):
    args = dict(name=f"tiny_mixed_{act}", act_dtype=act, expert_dtype=act, n_layers=2, canvas_len=40,
                head_dim=32, n_heads=2, prompt_len=100, batch=4, max_steps=6, seed=31,
                lm_scale=6.0 if act == "fp32" else 1.0)
    args.update(kw)
    return tiny_config(**args)


@pytest.mark.parametrize("act", ["fp32", "bf16"])
def test_mixed_tiny_matches_oracle(rt, act):
    """A prompt read into an empty cache, a canvas refined against a 100-row
    prompt, a canvas commit appended after 60 rows and a canvas refined with
    no prompt, interleaved, for three passes (the appends continue)."""
    cfg = _tiny_mix(rt, act)
    say(f"mixed batch, tiny {act}: append 37 | refine (P=100) | append 40 (P=60) | refine (P=0)")
    mix = Mix(rt, cfg, max_batch=2, max_tokens=80, kv_capacity=100 + 3 * 40 + 40)
    a0, r1 = Request(mix, 0, 0), Request(mix, 1, 100, seed=11)
    a2, r3 = Request(mix, 2, 60), Request(mix, 3, 0, seed=12, block=1)
    rng = np.random.default_rng(7)
    reps = []
    for p in range(3):
        say(f"  pass {p}")
        plan = [(a0, rng.integers(0, cfg.vocab, 37)), (r1, None), (a2, rng.integers(0, cfg.vocab, 40)), (r3, None)]
        reps += mix.run_pass(plan, 1e-5 if act == "fp32" else 1e-2)
    mix.close()
    assert_reports(cfg.replace(batch=1), reps)


def test_mixed_equals_separate_calls(rt):
    """fp32: each request's results from the mixed pass against the same
    request's own dg_denoise_step / dg_commit_canvas on the GPU (same inputs,
    different row stacking)."""
    cfg = _tiny_mix(rt, "fp32", name="tiny_mixed_vs_separate")
    say("mixed pass vs separate calls, fp32")
    mix = Mix(rt, cfg, max_batch=2, max_tokens=80, kv_capacity=200)
    a0, r1, a2, r3 = Request(mix, 0, 0), Request(mix, 1, 100, seed=11), Request(mix, 2, 60), \
        Request(mix, 3, 0, seed=12, block=1)
    rng = np.random.default_rng(9)
    t0 = torch.from_numpy(rng.integers(0, cfg.vocab, 37).astype(np.int32)).cuda()
    t2 = torch.from_numpy(rng.integers(0, cfg.vocab, 40).astype(np.int32)).cuda()
    rt_ = mix.rt
    sep = {}
    for name, req in (("r1", r1), ("r3", r3)):
        kv = rt_.KVCache(req.kv.k.clone(), req.kv.v.clone(), req.kv.length)
        cv = rt_.Canvas(req.canvas.tokens.clone(), req.canvas.committed.clone(), req.canvas.seed,
                        req.canvas.block, req.canvas.step)
        ent = torch.empty(1, cfg.canvas_len, device="cuda")
        am = torch.empty(1, cfg.canvas_len, dtype=torch.int32, device="cuda")
        rt_.denoise_step(mix.model, cv, kv, entropy=ent, argmax=am)
        sep[name] = (ent, am, cv)
    for name, req, t in (("a0", a0, t0), ("a2", a2, t2)):
        kv = rt_.KVCache(req.kv.k.clone(), req.kv.v.clone(), req.kv.length)
        rt_.commit_canvas(mix.model, t[None].contiguous(), kv)
        sep[name] = kv
    outs = {n: (torch.empty(cfg.canvas_len, device="cuda"),
                torch.empty(cfg.canvas_len, dtype=torch.int32, device="cuda")) for n in ("r1", "r3")}
    rt_.mixed_step(mix.model, [rt_.Append(a0.kv, t0), rt_.Refine(r1.kv, r1.canvas, *outs["r1"]),
                               rt_.Append(a2.kv, t2), rt_.Refine(r3.kv, r3.canvas, *outs["r3"])])
    torch.cuda.synchronize()
    for name, req in (("r1", r1), ("r3", r3)):
        ent, am, cv = sep[name]
        e_m, a_m = to_host(outs[name][0]), to_host(outs[name][1])
        dH = float(np.abs(e_m - to_host(ent)[0]).max())
        say(f"   {name}: max |dH| {dH:.2e}, argmax equal {int((a_m == to_host(am)[0]).sum())}/{cfg.canvas_len}")
        assert dH <= 1e-5
        np.testing.assert_array_equal(a_m, to_host(am)[0])
        np.testing.assert_array_equal(to_host(req.canvas.committed), to_host(cv.committed))
        np.testing.assert_array_equal(to_host(req.canvas.tokens), to_host(cv.tokens))
        assert req.canvas.step == cv.step == 1
    for name, req in (("a0", a0), ("a2", a2)):
        kv = sep[name]
        assert req.kv.length == kv.length
        n = kv.length
        for g, s in ((req.kv.k, kv.k), (req.kv.v, kv.v)):
            gg, ss = g[:, :, :, :n].double(), s[:, :, :, :n].double()
            rel = float((gg - ss).norm() / ss.norm())
            say(f"   {name}: cache rel-L2 {rel:.2e}")
            assert rel <= 1e-6
    mix.close()


def test_mixed_full_width_bf16(rt):
    """Full-width projections (d_model 2048, 16 x 128 heads, shared expert
    2048; 16 experts top-4, 8192 ids): two refine canvases of 200 (ragged
    tiles) against 300- and 0-row caches, a 70-token prompt read and a
    200-token canvas commit in one pass, two passes."""
    cfg = tiny_config(name="wide_mixed", n_layers=1, d_model=2048, n_heads=16, head_dim=128, n_experts=16,
                      top_k=4, d_expert=96, d_shared=2048, vocab=8192, canvas_len=200, max_steps=4,
                      prompt_len=300, batch=4, act_dtype="bf16", expert_dtype="bf16", seed=29, lm_scale=1.0)
    say("mixed batch, full width bf16: refine (P=300) | append 70 (P=0) | refine (P=0) | append 200 (P=300)")
    mix = Mix(rt, cfg, max_batch=2, max_tokens=400, kv_capacity=300 + 2 * 200)
    r0, a1 = Request(mix, 0, 300, seed=5), Request(mix, 1, 0)
    r2, a3 = Request(mix, 2, 0, seed=6, block=2), Request(mix, 3, 300)
    rng = np.random.default_rng(3)
    reps = []
    for p in range(2):
        say(f"  pass {p}")
        plan = [(r0, None), (a1, rng.integers(0, cfg.vocab, 70)), (r2, None), (a3, rng.integers(0, cfg.vocab, 200))]
        reps += mix.run_pass(plan, 1e-2)
    mix.close()
    del mix
    _free()
    assert_reports(cfg.replace(batch=1), reps)


def test_mixed_full_width_bf16_tall_segments(rt):
    """Four segments of 150 rows or more in one attention launch: three refine
    canvases of 200 against 300-, 0- and 500-row caches (300: a key tile spans
    cache and canvas rows) and a 150-token prompt read into a 120-row cache,
    750 rows a pass (large-M projection tiles), two passes.  (256-query tiles
    of 32-query waves, which win for a batch of canvases, measured 1.4 %
    slower here and are not used for segment tables.)"""
    cfg = tiny_config(name="wide_mixed_tall", n_layers=1, d_model=2048, n_heads=16, head_dim=128, n_experts=16,
                      top_k=4, d_expert=96, d_shared=2048, vocab=8192, canvas_len=200, max_steps=4,
                      prompt_len=500, batch=4, act_dtype="bf16", expert_dtype="bf16", seed=31, lm_scale=1.0)
    say("mixed batch, tall segments: refine (P=300) | refine (P=0) | append 150 (P=120) | refine (P=500)")
    mix = Mix(rt, cfg, max_batch=3, max_tokens=800, kv_capacity=500 + 2 * 200)
    r0, r1 = Request(mix, 0, 300, seed=7), Request(mix, 1, 0, seed=8, block=1)
    a2, r3 = Request(mix, 2, 120), Request(mix, 3, 500, seed=9, block=3)
    rng = np.random.default_rng(5)
    reps = []
    for p in range(2):
        say(f"  pass {p}")
        plan = [(r0, None), (r1, None), (a2, rng.integers(0, cfg.vocab, 150)), (r3, None)]
        reps += mix.run_pass(plan, 1e-2)
    mix.close()
    del mix
    _free()
    assert_reports(cfg.replace(batch=1), reps)


@pytest.mark.parametrize("act,n_append", [("fp32", 1100), ("bf16", 2100)])
def test_mixed_beyond_one_routed_launch(rt, act, n_append):
    """More rows than one routed-expert launch takes (1024 fp32, 2048 bf16):
    a long prompt read beside a refine canvas, so the experts run in two
    chunks and the refine rows sit in the first."""
    cfg = _tiny_mix(rt, act, name=f"tiny_mixed_long_{act}", batch=2, n_layers=2)
    say(f"mixed batch beyond one routed launch, {act}: refine (P=100) | append {n_append} (P=0)")
    mix = Mix(rt, cfg, max_batch=1, max_tokens=n_append + 40, kv_capacity=n_append + 100)
    r0, a1 = Request(mix, 0, 100, seed=13), Request(mix, 1, 0)
    rng = np.random.default_rng(11)
    reps = mix.run_pass([(r0, None), (a1, rng.integers(0, cfg.vocab, n_append))],
                        1e-5 if act == "fp32" else 1e-2)
    mix.close()
    assert_reports(cfg.replace(batch=1), reps)


def test_mixed_self_condition(rt):
    """Refine segments with self-conditioning in a mixed pass: from its second
    step each canvas's input carries its own previous predictions."""
    cfg = _tiny_mix(rt, "fp32", name="tiny_mixed_selfcond", self_condition=True)
    say("mixed batch with self-conditioning, fp32: refine (P=100) | append 30 | refine (P=0), 3 passes")
    mix = Mix(rt, cfg, max_batch=2, max_tokens=80, kv_capacity=220)
    r0, a1, r2 = Request(mix, 0, 100, seed=21), Request(mix, 1, 0), Request(mix, 2, 0, seed=22, block=1)
    rng = np.random.default_rng(13)
    reps = []
    for p in range(3):
        say(f"  pass {p}")
        reps += mix.run_pass([(r0, None), (a1, rng.integers(0, cfg.vocab, 30)), (r2, None)], 1e-5)
    mix.close()
    assert_reports(cfg.replace(batch=1), reps)


def test_mixed_sixteen_segments(rt):
    """The most segments a pass takes: four refine canvases and twelve appends
    of ragged lengths (1 to 64 tokens, some into empty caches), two passes."""
    cfg = _tiny_mix(rt, "fp32", name="tiny_mixed_16", batch=16, n_layers=1)
    say("mixed batch, 16 segments (4 refine + 12 appends of 1..64 tokens), fp32")
    mix = Mix(rt, cfg, max_batch=4, max_tokens=200, kv_capacity=100 + 2 * 64)
    refs = [Request(mix, i, 100 if i % 2 else 0, seed=30 + i, block=i) for i in range(4)]
    lens = [1, 3, 64, 17, 2, 40, 1, 33, 8, 64, 5, 11]
    apps = [Request(mix, 4 + i, (i * 13) % 100) for i in range(12)]
    rng = np.random.default_rng(17)
    reps = []
    for p in range(2):
        say(f"  pass {p}")
        plan = []
        for i in range(12):
            plan.append((apps[i], rng.integers(0, cfg.vocab, lens[(i + p) % 12])))
            if i % 3 == 2:
                plan.append((refs[i // 3], None))
        reps += mix.run_pass(plan, 1e-5)
    mix.close()
    assert_reports(cfg.replace(batch=1), reps)


@pytest.mark.parametrize("edt", ["fp8", "mxfp4", "mxfp4_a8"])
def test_mixed_low_precision_experts(rt, edt):
    """Mixed passes with fp8 (routed and shared), MXFP4 (routed) and MXFP4 x
    MXFP8 (routed; the token rows quantized by the RMSNorm of the stacked
    rows, d_model 128) experts: a prompt read, a refine canvas and a canvas
    commit, two passes."""
    extra = {"d_model": 128} if edt == "mxfp4_a8" else {}
    cfg = _tiny_mix(rt, "bf16", name=f"tiny_mixed_{edt}", expert_dtype=edt, d_expert=64, batch=3, **extra)
    say(f"mixed batch, {edt} experts: append 48 | refine (P=100) | append 40 (P=60)")
    mix = Mix(rt, cfg, max_batch=1, max_tokens=140, kv_capacity=100 + 2 * 48 + 40)
    a0, r1, a2 = Request(mix, 0, 0), Request(mix, 1, 100, seed=19), Request(mix, 2, 60)
    rng = np.random.default_rng(23)
    reps = []
    for p in range(2):
        say(f"  pass {p}")
        plan = [(a0, rng.integers(0, cfg.vocab, 48)), (r1, None), (a2, rng.integers(0, cfg.vocab, 40))]
        reps += mix.run_pass(plan, 1e-2)
    mix.close()
    assert_reports(cfg.replace(batch=1), reps)


def test_mixed_rejects_bad_segments(rt):
    """Validation happens before anything is enqueued; caller state is left as it was."""
    from diffusion_decoding_amd._lib import DGError
    cfg = _tiny_mix(rt, "fp32", name="tiny_mixed_errors")
    mix = Mix(rt, cfg, max_batch=1, max_tokens=100, kv_capacity=160)   # 100 rows a pass, 40 of them refine
    r0, a1 = Request(mix, 0, 100, seed=1), Request(mix, 1, 0)
    t = torch.zeros(10, dtype=torch.int32, device="cuda")
    cases = [
        ("two segments on one cache", [rt.Refine(r0.kv, r0.canvas), rt.Append(r0.kv, t)]),
        ("more refine rows than max_batch canvases",
         [rt.Refine(r0.kv, r0.canvas), rt.Refine(a1.kv, rt.Canvas.empty(1, cfg.canvas_len, 2))]),
        ("rows beyond the workspace", [rt.Refine(r0.kv, r0.canvas),
                                       rt.Append(a1.kv, torch.zeros(70, dtype=torch.int32, device="cuda"))]),
        ("append beyond capacity", [rt.Append(rt.KVCache(a1.kv.k, a1.kv.v, 155), t)]),
        ("no segments", []),
    ]
    for what, segs in cases:
        step = r0.canvas.step
        with pytest.raises(DGError):
            rt.mixed_step(mix.model, segs)
        say(f"   refused: {what}")
        assert r0.canvas.step == step and r0.kv.length == 100 and a1.kv.length == 0
    with pytest.raises(ValueError):
        rt.mixed_step(mix.model, [rt.Refine(r0.kv, rt.Canvas.empty(2, cfg.canvas_len, 3))])
    r0.canvas.step = cfg.max_steps
    with pytest.raises(DGError):
        rt.mixed_step(mix.model, [rt.Refine(r0.kv, r0.canvas)])
    mix.close()
