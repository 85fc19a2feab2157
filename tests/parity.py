"""Step-locked comparison of the HIP path against the oracle (test helper).

Each denoise step is checked three ways, all flags decided on oracle values:

(a) Backbone: the GPU's logits, final hidden rows and entropies against the
    oracle's own forward of the same canvas: logits rel-L2 <= 1e-4 (fp32
    workloads) or 2e-2 (bf16/fp8), entropy within h_tol().  Where two router
    logits of a row nearly tie in some layer (route_eps()), the GPU is made
    to take the oracle's expert picks for that row (a test hook), so every
    row stays compared.
(b) Decisions at the stated windows: the oracle's LM head, entropy, argmax,
    commit and re-noise applied to the GPU's own final hidden rows.  The GPU's
    argmax, commit mask and canvas must equal them bit for bit except where
    the top-2 logit gap is below 1e-3 or an entropy lies within 1e-4 nats of
    the commit cutoff or threshold; its entropies must lie within 1e-3 nats.
    The cutoff is the boundary the ranking draws: midway between the m-th and
    (m+1)-th smallest uncommitted entropy (none when every uncommitted
    position commits), so an entropy near it could fall on either side.
    At least half of the positions the step commits must be unflagged, so a
    run that flags everything fails.
(c) Decisions against the oracle's own forward, at windows() (the stated ones
    for fp32; wider for bf16/fp8, see below), with the counts reported.
After each step the GPU canvas is resynchronised to the oracle's state.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from oracle import model as om

ARGMAX_EPS = 1e-3
CUTOFF_EPS = 1e-4
H_TOL = 1e-3

# (c) compares decisions taken on two different forwards.  bf16/fp8 workloads
# carry a noise floor there that the stated windows do not cover: an
# activation whose exact value lies within the fp32-accumulation error
# (~1e-7 relative) of a bf16 rounding midpoint rounds the other way on the GPU
# than in the float64 oracle, moving that element by one bf16 ulp (2^-8
# relative); which elements flip depends on the summation order of every
# GEMM, so the floor is a property of the precision, not of one kernel (the
# unit tests show each kernel bit-exact away from rounding midpoints).
# Measured per step: at full width (d_model 2048, 262144 ids) logits rel-L2
# 1.1e-3 to 5.7e-3 at logit std ~1 (per-logit noise sigma up to ~6e-3) and
# |dH| up to 8.4e-4 nats; on the narrow test shapes (d_model 64 and 256, 512
# and 4096 ids) rel-L2 2e-3 to 3.5e-3 and |dH| up to 1.9e-3.  The top-2 gap
# is a difference of two noisy logits (sigma * sqrt(2) up to ~8e-3), so an
# argmax is ambiguous below about 2.5-3.5 of those: 2e-2.  An entropy 1e-4
# nats from the cutoff is likewise inside the |dH| floor, so the commit
# window is about 1.2-1.5x the largest |dH| seen.  An entropy averages the
# noise of all V logits, so its noise grows as V shrinks (about 1/sqrt(V)):
# at 262144 ids |dH| stays below 3e-4, at the 8192-id vocabularies of the
# full-width tests it reached 1.8e-3 (MXFP4 experts, two layers) and on the
# narrow shapes 1.9e-3; (c) takes 5e-3 nats.  The stated 1e-3 nats is held
# by (b), where both sides score the same hidden rows.  fp32 workloads carry
# no rounding points and keep the stated windows.
BF16_WIDE = dict(argmax=2e-2, cutoff=1e-3, h=5e-3)
BF16_NARROW = dict(argmax=2e-2, cutoff=2e-3, h=5e-3)


def windows(cfg) -> dict:
    if cfg.act_dtype == "fp32":
        return dict(argmax=ARGMAX_EPS, cutoff=CUTOFF_EPS, h=H_TOL)
    return BF16_WIDE if cfg.d_model >= 2048 else BF16_NARROW


def h_tol(cfg) -> float:
    return windows(cfg)["h"]


def logits_tol(cfg) -> float:
    return 1e-4 if cfg.act_dtype == "fp32" else 2e-2


# A router logit is an fp32 dot product; on bf16 workloads its inputs carry
# the rounding-flip noise above, so it moves by up to ~1e-3 between the two
# forwards (a top-k swap was observed at a 1.2e-3 gap between the k-th and
# (k+1)-th logit).  Rows with a gap below route_eps() in some layer take the
# oracle's picks on the GPU.  The GPU's own top-k is checked against the
# oracle on identical inputs by the router unit test (fp32 window 1e-5).
def route_eps(cfg) -> float:
    return 1e-5 if cfg.act_dtype == "fp32" else 5e-3


def forced_routing(trace: dict, cfg, B: int, N: int, rows_alloc: int) -> tuple[np.ndarray, int]:
    """[L, rows_alloc, k] int32: the oracle's expert ids of every row whose
    k-th and (k+1)-th router logits lie within route_eps() in that layer, -1
    elsewhere; and the number of distinct rows forced in some layer."""
    k, L = cfg.top_k, cfg.n_layers
    out = np.full((L, rows_alloc, k), -1, dtype=np.int32)
    rs, ids = trace.get("route_r32", []), trace.get("route_ids", [])
    per_canvas = len(rs) // B if B else 0
    any_row = np.zeros(B * N, dtype=bool)
    eps = route_eps(cfg)
    for b in range(B):
        for l in range(per_canvas):
            r = rs[b * per_canvas + l]
            if r.shape[1] <= k:
                continue
            srt = -np.sort(-r, axis=1)
            near = (srt[:, k - 1] - srt[:, k]) < eps
            rows = np.nonzero(near)[0]
            out[l, b * N + rows] = ids[b * per_canvas + l][rows]
            any_row[b * N + rows] = True
    return out, int(any_row.sum())


@dataclass
class StepReport:
    step: int
    # (a) backbone
    logits_rel: float = float("nan")
    hidden_rel: float = float("nan")
    max_dH: float = 0.0
    forced_rows: int = 0
    # (b) decisions from the GPU's hidden rows, stated windows
    max_dH_head: float = 0.0
    m: int = 0                    # positions the step commits (summed over canvases)
    checked_commits: int = 0      # of those, unflagged under (b)
    flagged_argmax_head: int = 0
    flagged_commit_head: int = 0
    mism_argmax_head: int = 0
    mism_commit_head: int = 0
    mism_tokens_head: int = 0
    # (c) decisions against the oracle's own forward
    flagged_argmax: int = 0
    flagged_commit: int = 0
    mism_argmax: int = 0
    mism_commit: int = 0
    mism_tokens: int = 0
    notes: list = field(default_factory=list)


def _rel(g, o) -> float:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-30))


def cut_boundary(H: np.ndarray, unc: np.ndarray, m: int) -> float:
    """Midpoint between the m-th and (m+1)-th smallest entropy among the
    uncommitted positions of one canvas (ties by position, NaN last); NaN when
    m is 0 or every uncommitted position commits."""
    idx = sorted(np.nonzero(unc)[0], key=lambda i: om._rank_key(float(H[i]), int(i)))
    if m <= 0 or m >= len(idx):
        return float("nan")
    return 0.5 * (float(H[idx[m - 1]]) + float(H[idx[m]]))


def _decision_flags(H, gap, cutoff, threshold, unc, argmax_eps, cutoff_eps):
    """(argmax flags, commit flags) on uncommitted rows."""
    fa = (gap < argmax_eps) & unc
    fc = np.zeros_like(unc)
    for b in range(H.shape[0]):
        if not np.isnan(cutoff[b]):
            fc[b] |= np.abs(H[b] - cutoff[b]) < cutoff_eps
        fc[b] |= np.abs(H[b] - threshold) < cutoff_eps
    return fa, fc & unc


def head_decisions(W, cfg, pre: "om.CanvasState", hidden: np.ndarray):
    """The oracle's LM head, confidence, commit and re-noise applied to the
    given final hidden rows [B, N, d] from the pre-step state: returns
    (H, argmax, gap, cutoff, state after the step, newly committed)."""
    B, N = pre.tokens.shape
    st = pre.copy()
    s = st.step
    Hs, As, Gs, cut = [], [], [], np.full(B, np.nan)
    newly = np.zeros((B, N), dtype=bool)
    for b in range(B):
        z = om.lm_head_logits(np.asarray(hidden[b], dtype=np.float64), W)
        H32, a, gap = om.confidence(z)
        unc = ~st.committed[b]
        cut[b] = cut_boundary(H32, unc, om.commit_count(int(unc.sum()), s, cfg.max_steps))
        newly[b] = om.commit_select(H32, a, st.tokens[b], st.committed[b], s, cfg.max_steps, cfg.threshold)
        Hs.append(H32); As.append(a); Gs.append(gap)
    for b in range(B):
        om.renoise(st.tokens[b], st.committed[b], st.seed, s, b, st.block, cfg.vocab,
                   getattr(cfg, "mask_token", -1))
    st.step = s + 1
    return np.stack(Hs), np.stack(As), np.stack(Gs), cut, st, newly


def compare_step(cfg, ores, pre, ost, gpu: dict, W=None) -> StepReport:
    """ores: the oracle's StepResult; pre / ost: its state before and after the
    step; gpu: host arrays (entropy, argmax, tokens, committed, and optionally
    logits and hidden [B*N, d]); W: oracle weights (needed for (b))."""
    B, N = ores.entropy.shape
    rep = StepReport(step=pre.step)
    unc = ~pre.committed
    # (a) backbone
    if gpu.get("logits") is not None and ores.logits is not None:
        rep.logits_rel = _rel(gpu["logits"].reshape(B, N, -1), ores.logits)
    if gpu.get("hidden") is not None and ores.hidden is not None:
        rep.hidden_rel = _rel(gpu["hidden"].reshape(B, N, -1), ores.hidden)
    dH = np.abs(gpu["entropy"].astype(np.float64) - ores.entropy)
    rep.max_dH = float(dH[unc].max()) if unc.any() else 0.0
    if unc.any():
        w = np.unravel_index(np.argmax(np.where(unc, dH, -1.0)), dH.shape)
        rep.notes.append(f"max dH at row {tuple(int(x) for x in w)}: top-2 gap {ores.gap[w]:.2e}")
    # (b) decisions from the GPU's own hidden rows
    if W is not None and gpu.get("hidden") is not None:
        hid = gpu["hidden"].reshape(B, N, -1)
        H, a, gap, cut, hst, newly = head_decisions(W, cfg, pre, hid)
        rep.max_dH_head = float(np.abs(gpu["entropy"].astype(np.float64) - H)[unc].max()) if unc.any() else 0.0
        fa, fc = _decision_flags(H, gap, cut, cfg.threshold, unc, ARGMAX_EPS, CUTOFF_EPS)
        rep.flagged_argmax_head, rep.flagged_commit_head = int(fa.sum()), int(fc.sum())
        rep.mism_argmax_head = int(((gpu["argmax"] != a) & unc & ~fa).sum())
        rep.mism_commit_head = int(((gpu["committed"].astype(bool) != hst.committed) & ~fc).sum())
        same = (gpu["committed"].astype(bool) == hst.committed) & ~(fa & hst.committed) & ~fc
        rep.mism_tokens_head = int(((gpu["tokens"] != hst.tokens) & same).sum())
        rep.m = int(newly.sum())
        rep.checked_commits = int((newly & ~fc & ~fa).sum())
    # (c) decisions against the oracle's own forward
    win = windows(cfg)
    ocut = np.array([cut_boundary(ores.entropy[b], unc[b], int(ores.m[b])) for b in range(B)])
    fa, fc = _decision_flags(ores.entropy, ores.gap, ocut, cfg.threshold, unc, win["argmax"], win["cutoff"])
    rep.flagged_argmax, rep.flagged_commit = int(fa.sum()), int(fc.sum())
    rep.mism_argmax = int(((gpu["argmax"] != ores.argmax) & unc & ~fa).sum())
    rep.mism_commit = int(((gpu["committed"].astype(bool) != ost.committed) & ~fc).sum())
    same = (gpu["committed"].astype(bool) == ost.committed) & ~(fa & ost.committed) & ~fc
    rep.mism_tokens = int(((gpu["tokens"] != ost.tokens) & same).sum())
    return rep


def assert_reports(cfg, reps, min_checked_frac: float = 0.5):
    for r in reps:
        if not np.isnan(r.logits_rel):
            assert r.logits_rel <= logits_tol(cfg), r
        assert r.max_dH <= h_tol(cfg), r
        assert r.mism_argmax == 0 and r.mism_commit == 0 and r.mism_tokens == 0, r
        assert r.max_dH_head <= H_TOL, r
        assert r.mism_argmax_head == 0 and r.mism_commit_head == 0 and r.mism_tokens_head == 0, r
        if r.m:
            assert r.checked_commits >= min_checked_frac * r.m, r


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()
