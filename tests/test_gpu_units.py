"""Kernel unit parity at full width: each phase of a block runs through its
dg_test_* entry (the same launches a denoise step makes) on inputs that are
the oracle's exact bf16 values, and is compared element by element with the
oracle's float64 result.  bf16 outputs must be the oracle's rounding except
within the stated fp32 error bound of a rounding boundary (tests/unit_ref.py
derives the bounds); fp32 outputs must lie within the bound; integer results
(top-k ids, the expert-major pair order) must be bit-exact except where two
router logits lie within the stated fp32 window (1e-5) of each other.

Shapes: the 2048-wide layer of the benchmark workloads -- a 256-token canvas
(batch 1), 1024 pooled tokens (batch 4) and a ragged 200-token canvas -- with
bf16 experts, fp8 E4M3 routed and shared experts, and MXFP4 routed experts at
the same width."""
import numpy as np
import pytest
import torch

from oracle import model as om
from oracle.numerics import round_bf16, round_fp32, round_mxfp8
from tests.gpu_helpers import say
from tests.parity import to_host
from tests.unit_ref import attention_ref, check_bf16, check_f32, gemm_tol, qkv_rope_ref, swiglu_ref
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu

ROUTER_EPS = 1e-5   # stated fp32 window for the router's top-k


@pytest.fixture(scope="module")
def rt():
    from diffusion_decoding_amd import runtime
    runtime._lib.load()
    return runtime


def _unit_cfg(kind: str):
    """One 2048-wide layer with a short vocabulary (the LM head is not used)."""
    if kind == "bf16":
        return get_config("c1").replace(name="unit_bf16", vocab=8192, batch=4, prompt_len=8192)
    if kind == "bf16_w1024":
        return get_config("c1").replace(name="unit_bf16_w1024", d_model=1024, n_heads=8, d_shared=1024,
                                        vocab=8192, batch=4, prompt_len=256)
    if kind == "fp8":
        return get_config("c4").replace(name="unit_fp8", n_layers=1, vocab=8192, n_canvases=1)
    if kind == "mxfp4":
        return get_config("c6").replace(name="unit_mxfp4", n_layers=1, vocab=8192, prompt_len=256)
    if kind == "mxfp4_a8":
        return get_config("c7").replace(name="unit_mxfp4_a8", n_layers=1, vocab=8192, prompt_len=256)
    raise ValueError(kind)


class Unit:
    def __init__(self, rt, kind: str, kv_capacity=None):
        self.rt = rt
        self.cfg = _unit_cfg(kind)
        say(f"[unit] inputs for {self.cfg.name}")
        self.inp = make_inputs(self.cfg, device="cuda", kv_capacity=kv_capacity)
        self.model = rt.Model(self.inp, max_batch=4, max_tokens=512)
        self.W = om.Weights(self.inp)

    def close(self):
        self.model.close()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def unit_bf16(rt):
    u = Unit(rt, "bf16", kv_capacity=8192 + 256)
    yield u
    u.close()


@pytest.fixture(scope="module")
def unit_bf16_w1024(rt):
    u = Unit(rt, "bf16_w1024")
    yield u
    u.close()


@pytest.fixture(scope="module")
def unit_fp8(rt):
    u = Unit(rt, "fp8")
    yield u
    u.close()


@pytest.fixture(scope="module")
def unit_mxfp4(rt):
    u = Unit(rt, "mxfp4")
    yield u
    u.close()


@pytest.fixture(scope="module")
def unit_mxfp4_a8(rt):
    u = Unit(rt, "mxfp4_a8")
    yield u
    u.close()


def _dev(x: np.ndarray) -> torch.Tensor:
    """bf16-valued float64 array -> bf16 device tensor (exact)."""
    assert np.array_equal(round_bf16(x), x)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


def _host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def _normed_rows(seed: int, T: int, d: int) -> np.ndarray:
    x = np.random.default_rng(seed).standard_normal((T, d))
    return round_bf16(om.rmsnorm(x, 1e-6))


def _report(what, nmis, nflag, total):
    say(f"   {what}: {nmis} of {total} differ from the oracle's rounding, {nflag} within the bound of a boundary")


# ----------------------------------------------------------------------------- QKV + RoPE

@pytest.mark.parametrize("B,n,pos0", [(1, 256, 1024), (4, 256, 8192), (1, 200, 300)])
def test_qkv_rope_unit(rt, unit_bf16, B, n, pos0):
    u, cfg = unit_bf16, unit_bf16.cfg
    H, dh = cfg.n_heads, cfg.head_dim
    say(f"QKV + RoPE unit: {B} x {n} rows at positions {pos0}..")
    a = _normed_rows(100 + B * n, B * n, cfg.d_model)
    q, k, v = rt.test_qkv_rope(u.model, 0, _dev(a), B, pos0)
    torch.cuda.synchronize()
    ref = qkv_rope_ref(a, u.W.dense(0, "wqkv"), B, n, H, dh, pos0, cfg.rope_theta)
    for name, got in (("q", q), ("k", k), ("v", v)):
        pre, tol, chk = ref[name]
        nmis, nflag = check_bf16(_host(got), pre, tol, f"{name} (B={B}, n={n})", mask=chk)
        _report(f"{name} ({int(chk.sum())} checked)", nmis, nflag, int(chk.sum()))


# ----------------------------------------------------------------------------- attention

def _bf16_normal(seed, shape):
    return round_bf16(np.random.default_rng(seed).standard_normal(shape))


# 4096 keys and more, or 64 canvas-heads and more, with 128 queries or more
# take the 32-query-wave kernel in 256-query tiles: batch 4 at 8192 and at
# 1024 cache rows, a ragged batch 2 whose cache length splits a key tile
# between cache and canvas rows and whose second query tile is part empty,
# causal commit passes into long caches and a causal batch-4 pass.  Fewer
# canvas-heads over 2048 keys or so take it in 128-query tiles with 4-8 key
# splits: one canvas over 2048 cache rows, a ragged 300-query canvas over a
# cache length that splits a key tile, a causal pass into 2000 rows and two
# canvases over 1500 rows.  Short ranges keep the 16-query waves.
@pytest.mark.parametrize("B,P,n,causal", [(1, 1024, 256, False), (4, 8192, 256, False), (1, 300, 200, False),
                                          (1, 512, 256, True), (2, 70, 200, True), (2, 4200, 300, False),
                                          (1, 4000, 256, True), (1, 4100, 200, True), (4, 1000, 256, False),
                                          (4, 300, 256, True), (1, 2048, 256, False), (1, 2100, 300, False),
                                          (1, 2000, 256, True), (2, 1500, 256, False)])
def test_attention_unit(rt, unit_bf16, B, P, n, causal):
    u, cfg = unit_bf16, unit_bf16.cfg
    H, dh = cfg.n_heads, cfg.head_dim
    say(f"attention unit: batch {B}, {P} cache rows, {n} queries, {'causal' if causal else 'bidirectional'}")
    q = _bf16_normal(200 + P, (B, H, n, dh))
    kc = _bf16_normal(201 + P, (B, H, n, dh))
    vc = _bf16_normal(202 + P, (B, H, n, dh))
    kvk, kvv = u.inp.kv_k[:, :B].clone(), u.inp.kv_v[:, :B].clone()
    if causal:
        # the new rows sit in the cache at [P, P + n), as a commit pass writes them
        kvk[0, :, :, P:P + n] = _dev(kc)
        kvv[0, :, :, P:P + n] = _dev(vc)
        kv = rt.KVCache(kvk, kvv, P)
        out = rt.test_attention(u.model, 0, _dev(q), kv)
    else:
        kv = rt.KVCache(kvk, kvv, P)
        out = rt.test_attention(u.model, 0, _dev(q), kv, _dev(kc), _dev(vc))
    torch.cuda.synchronize()
    got = _host(out).reshape(B, n, H, dh)
    cache_k = kvk[0].double().cpu().numpy()
    cache_v = kvv[0].double().cpu().numpy()
    pre = np.empty_like(got)
    tol = np.empty_like(got)
    for b in range(B):
        for h in range(H):
            if causal:
                K, V = cache_k[b, h, :P + n], cache_v[b, h, :P + n]
            else:
                K = np.concatenate([cache_k[b, h, :P], kc[b, h]])
                V = np.concatenate([cache_v[b, h, :P], vc[b, h]])
            o, t = attention_ref(q[b, h], K, V, causal_start=P if causal else None)
            pre[b, :, h], tol[b, :, h] = o, t
    nmis, nflag = check_bf16(got, pre, tol, f"attention B={B} P={P} n={n}")
    _report("attention output", nmis, nflag, got.size)


@pytest.mark.parametrize("P,n,causal", [(4200, 256, False), (4096, 160, True)])
def test_attention_unit_head_dim_64_long_keys(rt, P, n, causal):
    """head_dim 64 on the 32-query-wave kernel (4096 keys and more): a
    cache length that splits a key tile between cache and canvas rows, and a
    causal pass whose second query tile is part empty."""
    from workloads import tiny_config
    cfg = tiny_config(name="unit_dh64", d_model=256, n_heads=4, head_dim=64, n_experts=8, top_k=2, d_expert=64,
                      d_shared=64, vocab=512, canvas_len=256, prompt_len=P, act_dtype="bf16", expert_dtype="bf16",
                      seed=77)
    H, dh = cfg.n_heads, cfg.head_dim
    say(f"attention unit, head_dim 64: {P} cache rows, {n} queries, {'causal' if causal else 'bidirectional'}")
    inp = make_inputs(cfg, device="cuda", kv_capacity=P + 256)
    model = rt.Model(inp, max_batch=1, max_tokens=256)
    try:
        q = _bf16_normal(300 + P, (1, H, n, dh))
        kc = _bf16_normal(301 + P, (1, H, n, dh))
        vc = _bf16_normal(302 + P, (1, H, n, dh))
        kvk, kvv = inp.kv_k.clone(), inp.kv_v.clone()
        if causal:
            kvk[0, :, :, P:P + n] = _dev(kc)
            kvv[0, :, :, P:P + n] = _dev(vc)
            out = rt.test_attention(model, 0, _dev(q), rt.KVCache(kvk, kvv, P))
        else:
            out = rt.test_attention(model, 0, _dev(q), rt.KVCache(kvk, kvv, P), _dev(kc), _dev(vc))
        torch.cuda.synchronize()
        got = _host(out).reshape(1, n, H, dh)
        cache_k, cache_v = kvk[0].double().cpu().numpy(), kvv[0].double().cpu().numpy()
        pre, tol = np.empty_like(got), np.empty_like(got)
        for h in range(H):
            if causal:
                K, V = cache_k[0, h, :P + n], cache_v[0, h, :P + n]
            else:
                K = np.concatenate([cache_k[0, h, :P], kc[0, h]])
                V = np.concatenate([cache_v[0, h, :P], vc[0, h]])
            pre[0, :, h], tol[0, :, h] = attention_ref(q[0, h], K, V, causal_start=P if causal else None)
        nmis, nflag = check_bf16(got, pre, tol, f"attention dh 64 P={P} n={n}")
        _report("attention output", nmis, nflag, got.size)
    finally:
        model.close()
        torch.cuda.synchronize()


# ----------------------------------------------------------------------------- router

@pytest.mark.parametrize("T", [256, 1024])
def test_router_unit(rt, unit_bf16, T):
    """Router logits (fp32; at 256 rows they ride as extra tiles in the shared
    gate/up launch, at 1024 they have a launch of their own), top-k ids and
    weights."""
    u, cfg = unit_bf16, unit_bf16.cfg
    k = cfg.top_k
    say(f"router unit: {T} rows, {cfg.n_experts} experts, top-{k}")
    b = _normed_rows(300 + T, T, cfg.d_model)
    logits, ids, w = rt.test_router(u.model, 0, _dev(b))
    torch.cuda.synchronize()
    wr = u.W.dense(0, "wr")
    r = b @ wr.T
    ratio = check_f32(to_host(logits), r, gemm_tol(b, wr, r), "router logits")
    oids, ow = om.route(round_fp32(r), k)
    srt = -np.sort(-round_fp32(r), axis=1)
    tie = (srt[:, k - 1] - srt[:, k]) < ROUTER_EPS
    gi, gw = to_host(ids), to_host(w)
    ok = ~tie
    np.testing.assert_array_equal(gi[ok], oids[ok])
    np.testing.assert_allclose(gw[ok], ow[ok], rtol=0, atol=1e-6)
    say(f"   logits within {ratio:.2e} of the bound; {int(tie.sum())} rows with a near-tie (< {ROUTER_EPS}), "
        f"{int(ok.sum())} rows bit-exact ids")


# ----------------------------------------------------------------------------- shared expert

def _shared_case(rt, u, T):
    cfg = u.cfg
    b = _normed_rows(400 + T, T, cfg.d_model)
    hs, ys = rt.test_shared(u.model, 0, _dev(b))
    torch.cuda.synchronize()
    h_pre, h_tol = swiglu_ref(b, u.W.dense(0, "ws_gu"))
    nmis, nflag = check_bf16(_host(hs), h_pre, h_tol, "shared SwiGLU products")
    _report("shared h", nmis, nflag, h_pre.size)
    hg = _host(hs)
    wd = u.W.dense(0, "ws_d")
    ref = hg @ wd.T
    ratio = check_f32(to_host(ys), ref, gemm_tol(hg, wd, ref), "shared down (from the GPU's h)")
    say(f"   shared down within {ratio:.2e} of the bound")


@pytest.mark.parametrize("T", [256, 512, 1024])
def test_shared_unit_bf16(rt, unit_bf16, T):
    say(f"shared expert unit (bf16): {T} rows")
    _shared_case(rt, unit_bf16, T)


def test_shared_unit_fp8(rt, unit_fp8):
    say("shared expert unit (fp8 E4M3 weights, per-row scales): 256 rows")
    _shared_case(rt, unit_fp8, 256)


# ----------------------------------------------------------------------------- routed experts

def _moe_case(rt, u, b, ids, model=None):
    cfg = u.cfg
    T, k, E = ids.shape[0], cfg.top_k, cfg.n_experts
    h, y, pos = rt.test_moe(model or u.model, 0, _dev(b), torch.from_numpy(ids.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    hg, yg, pg = _host(h), to_host(y).astype(np.float64), to_host(pos)
    # pair order: expert-major, token-ascending (unique), bit-exact
    order = sorted(((int(ids[t, j]), t, j) for t in range(T) for j in range(k)))
    want = np.empty((T, k), dtype=np.int64)
    for r, (_, t, j) in enumerate(order):
        want[t, j] = r
    np.testing.assert_array_equal(pg, want)
    nmis = nflag = 0
    worst = 0.0
    a8 = cfg.expert_dtype == "mxfp4_a8"
    bq = round_mxfp8(b) if a8 else b        # the gate/up's token rows as the experts read them
    for e in range(E):
        ts, js = np.nonzero(ids == e)
        if ts.size == 0:
            continue
        w_gu, w_d = u.W.expert(0, e)
        rows = pg[ts, js]
        h_pre, h_tol = swiglu_ref(bq[ts], w_gu, scaled_mfma=a8)
        a, f = check_bf16(hg[rows], h_pre, h_tol, f"expert {e} SwiGLU products", max_frac=1.0)
        nmis, nflag = nmis + a, nflag + f
        ref = hg[rows] @ w_d.T
        worst = max(worst, check_f32(yg[rows], ref, gemm_tol(hg[rows], w_d, ref), f"expert {e} down"))
    # (the scaled MFMA's looser accumulation leaves more products next to a
    # rounding boundary; every difference is still within the bound)
    assert nmis <= (5e-2 if a8 else 5e-3) * hg.size, nmis
    _report("routed h", nmis, nflag, hg.size)
    say(f"   routed down (from the GPU's h) within {worst:.2e} of the bound")


def _oracle_ids(u, b):
    r32 = round_fp32(b @ u.W.dense(0, "wr").T)
    ids, _ = om.route(r32, u.cfg.top_k)
    return ids


@pytest.mark.parametrize("T", [256, 383, 384, 512, 1024, 2048])
def test_moe_unit_bf16(rt, unit_bf16, T):
    """256 rows: about 16 pairs per expert, one weight-stream pass each; 383
    and 384 rows: either side of the switch to grouped tiles (24 pairs per
    expert on average), the weight stream's further passes spread over the
    grid, then the routing permutation and the grouped gate/up; 512 rows:
    32 pairs per expert on the grouped gate/up (128-pair tiles a quarter
    full) and the weight-stream down; 1024
    rows (four canvases pooled): about 64 pairs per expert, the grouped gate/up
    (128-pair tiles) and the pooled 96-token down passes; 2048 rows: about 128
    pairs per expert, the grouped gate/up and down (an expert over one or two
    pair tiles)."""
    say(f"routed experts unit (bf16): {T} rows, routing from the oracle's router")
    b = _normed_rows(500 + T, T, unit_bf16.cfg.d_model)
    _moe_case(rt, unit_bf16, b, _oracle_ids(unit_bf16, b))


def test_moe_unit_bf16_pooled_narrow(rt, unit_bf16_w1024):
    """d_model 1024, where the grouped tiles (K = 2048) do not apply: 1024
    rows put about 64 pairs on an expert, so both routed kernels take the
    pooled weight stream -- 96-token passes, the gate/up staging its token
    rows in 256-column chunks, the down staging whole 704-wide h rows."""
    say("routed experts unit (bf16, d_model 1024): 1024 pooled rows")
    b = _normed_rows(1500, 1024, unit_bf16_w1024.cfg.d_model)
    _moe_case(rt, unit_bf16_w1024, b, _oracle_ids(unit_bf16_w1024, b))


@pytest.fixture(scope="module")
def wide_model(rt, unit_bf16):
    """The bf16 unit layer with room for 8192 rows per call."""
    model = rt.Model(unit_bf16.inp, max_batch=16, max_tokens=512)
    yield model
    model.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [4096, 8192])
def test_moe_unit_bf16_many_rows(rt, unit_bf16, wide_model, T):
    """More rows than the one-workgroup routing permutation takes (2048): 256
    and 512 pairs per expert in one routed launch -- the three-launch
    permutation, the grouped gate/up and the grouped down."""
    say(f"routed experts unit (bf16): {T} rows in one launch, routing from the oracle's router")
    b = _normed_rows(700 + T, T, unit_bf16.cfg.d_model)
    _moe_case(rt, unit_bf16, b, _oracle_ids(unit_bf16, b), model=wide_model)


@pytest.mark.parametrize("T", [256, 1536])
def test_moe_unit_bf16_skewed(rt, unit_bf16, T):
    """Every row routed to the same 8 experts (as when every open position
    holds the same token).  256 rows: 256 pairs on each, eight 32-token
    passes, the third and later spread over the grid; 1536 rows: the grouped
    gate/up, twelve 128-pair tiles on each of the 8 experts, none on the rest."""
    say(f"routed experts unit (bf16): {T} rows all on experts 3, 10, .., 52")
    cfg = unit_bf16.cfg
    b = _normed_rows(600, T, cfg.d_model)
    ids = np.tile(np.array([3 + 7 * j for j in range(cfg.top_k)]), (T, 1))
    _moe_case(rt, unit_bf16, b, ids)


def test_moe_unit_fp8(rt, unit_fp8):
    """fp8 E4M3 routed experts at full width: 16 codes per lane-load in both
    the gate/up (K = 2048) and the down kernel (K = d_expert = 704)."""
    say("routed experts unit (fp8): 256 rows")
    b = _normed_rows(700, 256, unit_fp8.cfg.d_model)
    _moe_case(rt, unit_fp8, b, _oracle_ids(unit_fp8, b))


def test_moe_unit_mxfp4(rt, unit_mxfp4):
    """MXFP4 routed experts at full width: 32 codes per lane-load and one E8M0
    scale per lane in the gate/up kernel (K = 2048), 16 codes in the down
    kernel (K = d_expert = 704)."""
    say("routed experts unit (MXFP4): 256 rows")
    b = _normed_rows(800, 256, unit_mxfp4.cfg.d_model)
    _moe_case(rt, unit_mxfp4, b, _oracle_ids(unit_mxfp4, b))


@pytest.mark.parametrize("T", [256, 1024, 2048])
def test_moe_unit_mxfp4_a8(rt, unit_mxfp4_a8, T):
    """MXFP4 weights x MXFP8 token rows on the scaled MFMA (gate/up, K =
    2048): the rows are quantized while staged (one E8M0 scale per 32), 32
    tokens per pass; 1024 and 2048 rows put 64 and 128 pairs on an expert, so
    its further passes spread over the grid.  The down reads bf16 h."""
    say(f"routed experts unit (MXFP4 x MXFP8): {T} rows")
    b = _normed_rows(900 + T, T, unit_mxfp4_a8.cfg.d_model)
    _moe_case(rt, unit_mxfp4_a8, b, _oracle_ids(unit_mxfp4_a8, b))


def test_moe_unit_mxfp4_pooled(rt, unit_mxfp4):
    """1024 pooled rows, about 64 pairs per expert: MXFP4 gate/up passes of 48
    tokens with chunked staging (most experts take two, in their own
    workgroups); the down's 96-token passes."""
    say("routed experts unit (MXFP4): 1024 pooled rows (48-token gate/up passes)")
    b = _normed_rows(801, 1024, unit_mxfp4.cfg.d_model)
    _moe_case(rt, unit_mxfp4, b, _oracle_ids(unit_mxfp4, b))


def _mx8_rows(seed: int, rows: int, d: int) -> np.ndarray:
    """bf16 rows that reach every branch of the MXFP8 conversion: random
    values over 2^-40 .. 2^40, zero and negative-zero blocks, halfway cases
    of the E4M3 grid, block maxima that round past 448, elements on the
    subnormal grid, bf16 subnormals and very large magnitudes."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, d)) * np.exp2(g.integers(-40, 40, (rows, d // 32, 1))).repeat(32, -1).reshape(rows, d)
    x[0, :32] = 0.0
    x[0, 32:64] = -0.0
    x[1, :32] = np.array([1.0 + 1 / 16, 1.0 + 3 / 16, -(1.0 + 5 / 16), 2.0 ** -7 * 1.5] + [0.01] * 28)
    x[1, 0:32] *= 2.0 ** -8                   # block max 1.0625 * 2^-8: scale 2^-16, halfway cases stay halfway
    x[1, 32:64] = 1.9 * 2.0 ** 5              # amax 1.9 * 2^5 -> 486.4 / 448 after scaling: clamped
    x[1, 64:96] = g.standard_normal(32) * 2.0 ** -120
    x[1, 96:128] = np.where(g.random(32) < 0.5, 1e-39, -3e-40)    # bf16 subnormals
    x[2, :32] = g.standard_normal(32) * 1e30
    x[2, 32:64] = np.concatenate([[300.0], g.standard_normal(31) * 2.0 ** -12])  # small ones on the subnormal grid
    return round_bf16(x)


@pytest.mark.parametrize("norm", [False, True])
def test_mx8_quantize_bit_exact(rt, norm):
    """The MXFP8 conversion of bf16 rows (standalone, and fused into the
    RMSNorm whose output the MXFP4 x MXFP8 gate/up reads) gives the oracle's
    E4M3 codes and E8M0 scales bit for bit."""
    from oracle.numerics import quantize_mxfp8
    say(f"MXFP8 quantization ({'fused into RMSNorm' if norm else 'standalone'}): 64 x 2048 rows")
    x = _mx8_rows(31, 64, 2048)
    xt = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda()
    codes, scales, y = rt.test_mx8_quantize(xt, 1e-6 if norm else None)
    torch.cuda.synchronize()
    src = _host(y) if norm else x
    want_c, want_s = quantize_mxfp8(src)
    np.testing.assert_array_equal(to_host(scales), want_s)
    np.testing.assert_array_equal(to_host(codes), want_c)
    say(f"   {codes.numel()} codes and {scales.numel()} scales bit-exact")


def test_fp4_decode_exhaustive(rt):
    """Every byte (two E2M1 codes) under E8M0 scale codes from 2^-90 to 2^100:
    the widening the MXFP4 kernels use equals the oracle's decode rounded to
    bf16 (exactly representable) wherever the product is a normal bf16 number."""
    from oracle.numerics import decode_mxfp4
    codes = np.arange(256, dtype=np.uint8)
    scale_codes = np.array([37, 64, 100, 118, 121, 125, 126, 127, 128, 131, 160, 200, 227], dtype=np.uint8)
    packed = np.tile(codes, len(scale_codes))                      # 16 blocks of 16 bytes per scale code
    scales = np.repeat(scale_codes, 16)
    got = rt.test_fp4_decode(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    ref = decode_mxfp4(packed.reshape(-1, 16), scales.reshape(-1, 1)).reshape(-1)
    g = _host(got)
    normal = (np.abs(ref) >= 2.0 ** -126) & (np.abs(ref) < 2.0 ** 127)
    np.testing.assert_array_equal(round_bf16(ref[normal]), ref[normal])
    np.testing.assert_array_equal(g[normal], ref[normal])
    assert not g[ref == 0].any()
    say(f"   {int(normal.sum())} decoded values bit-exact; {int((ref == 0).sum())} zeros")
