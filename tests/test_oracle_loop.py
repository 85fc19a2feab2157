"""Oracle pins for commit selection, re-noising, the denoise loop and the
causal commit pass: brute force on tiny cases, invariants the pages fix
(committed tokens are locked, every position is committed by the step cap),
closed forms, and end-to-end symmetries."""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import model as om
from oracle import philox
from workloads import get_config, make_inputs, tiny_config

RNG = np.random.default_rng(5)


def _count_rank_commit(H32, a, tok, committed, s, S, thr):
    """Commit rule restated as counting: i commits iff fewer than m uncommitted
    positions precede it in (entropy, index) order, or its entropy is below thr."""
    n = len(tok)
    unc = [i for i in range(n) if not committed[i]]
    m = math.ceil(len(unc) / (S - s)) if unc else 0
    tok, committed = tok.copy(), committed.copy()
    for i in unc:
        before = sum(1 for j in unc if (H32[j] < H32[i]) or (H32[j] == H32[i] and j < i))
        if before < m or H32[i] < thr:
            tok[i], committed[i] = a[i], True
    return tok, committed


def test_commit_select_brute_force_with_ties():
    for trial in range(300):
        n = int(RNG.integers(1, 24))
        S = int(RNG.integers(1, 9))
        s = int(RNG.integers(0, S))
        H = RNG.integers(0, 5, n) * 0.5                 # many exact ties
        committed = RNG.random(n) < 0.3
        tok = RNG.integers(0, 100, n)
        a = RNG.integers(100, 200, n)
        thr = [-np.inf, 1.0, 0.75][trial % 3]
        want_tok, want_c = _count_rank_commit(H, a, tok, committed, s, S, thr)
        t2, c2 = tok.copy(), committed.copy()
        newly = om.commit_select(H, a, t2, c2, s, S, thr)
        np.testing.assert_array_equal(t2, want_tok)
        np.testing.assert_array_equal(c2, want_c)
        np.testing.assert_array_equal(newly, c2 & ~committed)


def test_commit_nan_entropy_ranks_last_and_never_passes_threshold():
    H = np.array([np.nan, 0.5, np.nan, 2.0])
    tok, c = np.zeros(4, np.int64), np.zeros(4, bool)
    om.commit_select(H, np.arange(4) + 10, tok, c, 0, 2, 1.0)   # m = 2
    np.testing.assert_array_equal(c, [False, True, False, True])


def test_commit_schedule_without_threshold_hits():
    for N, S, expect in [(16, 8, [2] * 8), (256, 48, [6] * 16 + [5] * 32)]:
        U, got = N, []
        for s in range(S):
            m = om.commit_count(U, s, S)
            got.append(m)
            U -= m
        assert got == expect and U == 0


def test_last_step_commits_everything():
    H = RNG.standard_normal(10) + 5
    tok, c = np.zeros(10, np.int64), np.zeros(10, bool)
    c[:3] = True
    om.commit_select(H, np.arange(10), tok, c, 7, 8, 1.0)
    assert c.all()


def test_renoise_touches_only_uncommitted_and_uses_step_counter():
    tok = np.arange(32)
    committed = RNG.random(32) < 0.5
    before = tok.copy()
    om.renoise(tok, committed, 77, 3, 1, 2, 512)
    np.testing.assert_array_equal(tok[committed], before[committed])
    idx = np.nonzero(~committed)[0]
    np.testing.assert_array_equal(tok[idx], philox.canvas_draw(77, idx, 4, 1, 2, 512))


# ----------------------------------------------------------------------------- full loop

def _setup(cfg):
    inp = make_inputs(cfg)
    W = om.Weights(inp, cache=True)
    kv = om.KV(inp.kv_k, inp.kv_v, inp.kv_len, bf16=cfg.act_dtype == "bf16")
    return inp, W, kv


@pytest.mark.parametrize("cfg", [get_config("c0"), tiny_config(threshold=-math.inf, seed=11),
                                 tiny_config(act_dtype="bf16", expert_dtype="bf16", seed=12),
                                 tiny_config(batch=3, seed=13)])
def test_loop_invariants(cfg):
    inp, W, kv = _setup(cfg)
    hist = []

    def hook(res, st):
        hist.append((st.tokens.copy(), st.committed.copy(), res))
    state, steps = om.generate_canvas(W, kv, cfg, cfg.seed, hook=hook)
    assert 1 <= steps <= cfg.max_steps
    assert state.committed.all()
    prev_tok = prev_c = None
    for s, (tok, com, res) in enumerate(hist):
        B = tok.shape[0]
        if prev_c is not None:
            assert (com >= prev_c).all()                          # monotone mask
            np.testing.assert_array_equal(tok[prev_c], prev_tok[prev_c])   # locked tokens
        for b in range(B):
            U = int((~(prev_c[b] if prev_c is not None else np.zeros_like(com[b]))).sum())
            m = om.commit_count(U, s, cfg.max_steps)
            assert res.newly[b].sum() >= min(U, m)
            # committed values are the step's argmax
            np.testing.assert_array_equal(tok[b][res.newly[b]], res.argmax[b][res.newly[b]])
        prev_tok, prev_c = tok, com
    if cfg.threshold == -math.inf:
        assert steps == cfg.max_steps
        assert [int(r.newly.sum()) for _, _, r in hist] == [2 * cfg.batch] * cfg.max_steps
    np.testing.assert_array_equal(state.tokens, hist[-1][0])


def _fim_mask(B, N, head, tail):
    """Known prefix and suffix, open middle (fill-in-the-middle)."""
    m = np.zeros((B, N), dtype=bool)
    m[:, :head] = True
    m[:, N - tail:] = True
    return m


@pytest.mark.parametrize("cfg", [tiny_config(threshold=-math.inf, seed=31),
                                 tiny_config(batch=2, seed=32)])
def test_prefill_positions_are_fixed_and_only_open_ones_are_scheduled(cfg):
    """Pre-committed positions keep their tokens through the loop; the commit
    count follows ceil(U / (S_max - s)) over the open positions only, and every
    open position is committed by the step cap."""
    inp, W, kv = _setup(cfg)
    B, N = cfg.batch, cfg.canvas_len
    mask = _fim_mask(B, N, 5, 3)
    given = np.random.default_rng(3).integers(0, cfg.vocab, (B, N))
    st = om.prefill(om.init_state(cfg, cfg.seed), given, mask)
    np.testing.assert_array_equal(st.tokens[mask], given[mask])
    init = om.init_state(cfg, cfg.seed)
    np.testing.assert_array_equal(st.tokens[~mask], init.tokens[~mask])   # open ones keep their draw
    hist = []
    state, steps = om.generate_canvas(W, kv, cfg, cfg.seed, state=st,
                                      hook=lambda res, s: hist.append((s.committed.copy(), res)))
    assert state.committed.all()
    np.testing.assert_array_equal(state.tokens[mask], given[mask])
    prev = mask.copy()
    for s, (com, res) in enumerate(hist):
        assert not (res.newly & mask).any()                    # never re-selected
        for b in range(B):
            U = int((~prev[b]).sum())
            assert res.m[b] == om.commit_count(U, s, cfg.max_steps)
            assert res.newly[b].sum() >= min(U, res.m[b])
        prev = com
    if cfg.threshold == -math.inf:
        # 8 open positions over 8 steps: one per step
        assert steps == cfg.max_steps
        assert [int(r.newly.sum()) for _, r in hist] == [B] * cfg.max_steps


def test_prefill_of_every_position_stops_after_one_step_unchanged():
    cfg = tiny_config(seed=33)
    inp, W, kv = _setup(cfg)
    given = np.arange(cfg.canvas_len)[None, :] % cfg.vocab
    st = om.prefill(om.init_state(cfg, cfg.seed), given, np.ones((1, cfg.canvas_len), bool))
    state, steps = om.generate_canvas(W, kv, cfg, cfg.seed, state=st)
    assert steps == 1
    np.testing.assert_array_equal(state.tokens, given)


def test_prefill_equals_the_same_canvas_committed_by_hand():
    """A prefilled canvas is the state a loop would be in had those positions
    been committed: a step from either gives the same result."""
    cfg = tiny_config(seed=34)
    inp, W, kv = _setup(cfg)
    mask = _fim_mask(1, cfg.canvas_len, 4, 4)
    given = (np.arange(cfg.canvas_len) * 7 % cfg.vocab)[None, :]
    a = om.prefill(om.init_state(cfg, cfg.seed), given, mask)
    b = om.init_state(cfg, cfg.seed)
    b.tokens[mask] = given[mask]
    b.committed[mask] = True
    ra = om.denoise_step(W, kv, a, cfg)
    rb = om.denoise_step(W, kv, b, cfg)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.committed, b.committed)
    np.testing.assert_array_equal(ra.entropy, rb.entropy)
    with pytest.raises(ValueError):
        om.prefill(a, given, mask)          # only before the first step


def test_c0_exercises_threshold_early_stop():
    cfg = get_config("c0")
    inp, W, kv = _setup(cfg)
    _, steps = om.generate_canvas(W, kv, cfg, cfg.seed)
    assert steps < cfg.max_steps


def test_resume_is_bit_exact():
    cfg = tiny_config(threshold=0.3, seed=21)
    inp, W, kv = _setup(cfg)
    full, n_full = om.generate_canvas(W, kv, cfg, cfg.seed)
    st = om.init_state(cfg, cfg.seed)
    om.denoise_step(W, kv, st, cfg)
    om.denoise_step(W, kv, st, cfg)
    saved = st.copy()
    resumed, n_res = om.generate_canvas(W, kv, cfg, cfg.seed, state=saved)
    assert n_res == n_full
    np.testing.assert_array_equal(resumed.tokens, full.tokens)


def test_step_is_permutation_equivariant_without_rope():
    cfg = tiny_config(rope_theta=0.0, seed=31)
    inp, W, kv = _setup(cfg)
    st = om.init_state(cfg, cfg.seed)
    perm = RNG.permutation(cfg.canvas_len)
    st2 = st.copy()
    st2.tokens = st.tokens[:, perm].copy()
    r1 = om.denoise_step(W, kv, st, cfg)
    r2 = om.denoise_step(W, kv, st2, cfg)
    np.testing.assert_allclose(r2.entropy, r1.entropy[:, perm], rtol=1e-6)
    np.testing.assert_array_equal(r2.argmax, r1.argmax[:, perm])


def test_step_reduces_to_embedding_lm_head_when_blocks_are_zero():
    cfg = tiny_config(seed=41)
    inp = make_inputs(cfg)
    for name in ("wo", "w_d", "ws_d"):
        inp.layers[0][name].zero_()
    W = om.Weights(inp, cache=True)
    kv = om.KV(inp.kv_k, inp.kv_v, inp.kv_len, bf16=False)
    st = om.init_state(cfg, cfg.seed)
    tok0 = st.tokens.copy()
    res = om.denoise_step(W, kv, st, cfg, keep_logits=True)
    x = inp.embed.double()[torch.from_numpy(tok0[0])]
    hf = torch.nn.functional.rms_norm(x, (cfg.d_model,), eps=cfg.rms_eps)
    z = (hf @ inp.lm_head.double().T).numpy()
    np.testing.assert_allclose(res.logits[0], z, rtol=1e-10, atol=1e-10)
    ent = scipy.stats.entropy(scipy.special.softmax(z, axis=1), axis=1)
    np.testing.assert_allclose(res.entropy[0], ent, rtol=1e-6)


def test_canvas_init_is_philox_tag_zero():
    cfg = tiny_config(batch=2, seed=51)
    st = om.init_state(cfg, 999, block=3)
    for b in range(2):
        np.testing.assert_array_equal(
            st.tokens[b], philox.canvas_draw(999, np.arange(cfg.canvas_len), 0, b, 3, cfg.vocab))


# ----------------------------------------------------------------------------- commit pass

@pytest.mark.parametrize("act", ["fp32", "bf16"])
def test_commit_pass_equals_token_by_token_append(act):
    cfg = tiny_config(n_layers=2, act_dtype=act, expert_dtype=act, seed=61,
                      prompt_mode="tokens", prompt_len=8, n_canvases=1)
    inp = make_inputs(cfg)
    W = om.Weights(inp, cache=True)
    toks = RNG.integers(0, cfg.vocab, (1, 12))
    kv_a = om.KV(inp.kv_k, inp.kv_v, 0, bf16=act == "bf16")
    om.commit_canvas(W, kv_a, toks, cfg)
    kv_b = om.KV(inp.kv_k, inp.kv_v, 0, bf16=act == "bf16")
    for i in range(12):
        om.commit_canvas(W, kv_b, toks[:, i:i + 1], cfg)
    assert kv_a.length == kv_b.length == 12
    tol = dict(rtol=1e-10, atol=1e-10) if act == "fp32" else dict(rtol=2e-2, atol=2e-2)
    np.testing.assert_allclose(kv_a.k[:, :, :, :12].double().numpy(),
                               kv_b.k[:, :, :, :12].double().numpy(), **tol)
    np.testing.assert_allclose(kv_a.v[:, :, :, :12].double().numpy(),
                               kv_b.v[:, :, :, :12].double().numpy(), **tol)


def test_commit_pass_single_token_equals_bidirectional_layer():
    cfg = tiny_config(n_layers=1, seed=71)
    inp, W, kv = _setup(cfg)
    prec = om.Prec("fp32")
    x = W.embed_rows(np.array([5]))
    kvk, kvv = kv.get(0, 0)
    xb, kb, vb = om.layer_forward(x, W, 0, kvk, kvv, kv.length, prec, cfg, causal=False)
    xc, kc, vc = om.layer_forward(x, W, 0, kvk, kvv, kv.length, prec, cfg, causal=True)
    np.testing.assert_array_equal(xb, xc)
    np.testing.assert_array_equal(kb, kc)


def test_commit_pass_capacity_error():
    cfg = tiny_config(prompt_mode="tokens", prompt_len=8, n_canvases=1, seed=81)
    inp = make_inputs(cfg)
    W = om.Weights(inp)
    kv = om.KV(inp.kv_k, inp.kv_v, 0, bf16=False)
    with pytest.raises(ValueError):
        om.commit_canvas(W, kv, np.zeros((1, cfg.kv_capacity + 1), np.int64), cfg)


def test_block_generate_tiny():
    cfg = tiny_config(prompt_mode="tokens", prompt_len=8, n_canvases=3, seed=91)
    inp = make_inputs(cfg)
    W = om.Weights(inp, cache=True)
    kv = om.KV(inp.kv_k, inp.kv_v, 0, bf16=False)
    outs, steps = om.block_generate(W, kv, cfg, inp.prompt_tokens.numpy().astype(np.int64))
    assert kv.length == 8 + 3 * cfg.canvas_len
    assert len(outs) == 3 and all(1 <= s <= cfg.max_steps for s in steps)


# ----------------------------------------------------------------------------- absorbing-state noise

def test_absorbing_noise_masks_every_open_position():
    """Masked-diffusion variant (a [MASK] id instead of uniform draws), with
    the threshold off so the schedule runs to the cap: the canvas starts as all
    [MASK], after every step each uncommitted position holds [MASK] again,
    committed tokens never change and are that step's argmax, and each step
    commits exactly ceil(U / (S_max - s))."""
    cfg = tiny_config(batch=2, seed=61, mask_token=511, threshold=-math.inf)
    inp, W, kv = _setup(cfg)
    st = om.init_state(cfg, cfg.seed)
    assert (st.tokens == 511).all() and not st.committed.any()
    prev_tok, prev_com = st.tokens.copy(), st.committed.copy()
    after = []
    state, steps = om.generate_canvas(W, kv, cfg, cfg.seed, state=st,
                                      step_hook=lambda res, s: after.append((s.tokens.copy(), s.committed.copy(), res)))
    assert state.committed.all() and steps == cfg.max_steps == len(after)
    for s, (tok, com, res) in enumerate(after):
        assert (tok[~com] == 511).all()                                   # re-masked
        np.testing.assert_array_equal(tok[prev_com], prev_tok[prev_com])  # locked
        np.testing.assert_array_equal(com, prev_com | res.newly)
        np.testing.assert_array_equal(tok[res.newly], res.argmax[res.newly])
        for b in range(cfg.batch):
            U = int((~prev_com[b]).sum())
            assert res.newly[b].sum() == om.commit_count(U, s, cfg.max_steps)
        prev_tok, prev_com = tok, com


def test_absorbing_first_step_sees_identical_rows_without_rope():
    """With RoPE off and every position holding [MASK], every canvas row is the
    same input, so the first step gives every position the same prediction
    and commits exactly ceil(N / S_max) of them (threshold off), all with that
    token."""
    cfg = tiny_config(rope_theta=0.0, threshold=-math.inf, seed=62, mask_token=7)
    inp, W, kv = _setup(cfg)
    st = om.init_state(cfg, cfg.seed)
    res = om.denoise_step(W, kv, st, cfg)
    H, a = res.entropy[0], res.argmax[0]
    assert (a == a[0]).all()
    np.testing.assert_allclose(H, H[0], rtol=1e-9)
    m = om.commit_count(cfg.canvas_len, 0, cfg.max_steps)
    assert res.newly[0].sum() == m == math.ceil(cfg.canvas_len / cfg.max_steps)
    assert (st.tokens[0][res.newly[0]] == a[0]).all()
    assert (st.tokens[0][~res.newly[0]] == 7).all()


def test_uniform_noise_is_the_default():
    cfg = tiny_config(seed=63)
    assert cfg.mask_token == -1
    st = om.init_state(cfg, cfg.seed)
    np.testing.assert_array_equal(st.tokens[0], om.canvas_init(cfg.seed, cfg.canvas_len, 0, 0, cfg.vocab))
