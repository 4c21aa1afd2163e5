"""CPU oracle for the PD-guided mixed-precision bit allocation.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module; the
product (libddg.so) shares no code with it.

Source: [WDQ] the Wan-Dancer-14B mixed-precision quantization report
(www.mtrt.cn), §3.2 "PD-Guided Mixed Precision Bit Allocation": minimise the
parameter-weighted sum of the tensors' quantization errors
||W_i - Q_{b_i}(W_i)||_F^2 subject to a target average bit width, by a
continuous relaxation -- one parameter per tensor mapped through a sigmoid
onto [b_min, b_max], a temperature-annealed softmax over the candidate widths
that blends each tensor's error table, a Lagrange term plus a quadratic
penalty 1e4 (bpw - target)^2 on the budget -- with random restarts, then
rounding and keeping the best restart.  §4.4 and §4.6 report its results.

Readings where the section is silent:

R7   Candidate widths are the packable ones, 3..7; b_min = 3, b_max = 7.
R8   dist(b, c) = |b - c|; the soft weights are softmax_c(-|b - c| / temp),
     temp = max(2 (1 - it / iters), 0.05).
R9   The error table enters normalised: per-weight MSE of tensor i at width
     c, divided by the parameter-weighted MSE of the uniform allocation at the
     candidate nearest the target (lower on ties), times 100 -- the error term
     is in percent of the uniform allocation's error.  Raw per-weight MSEs
     (~1e-7 for DiT weights) vanish next to the 1e4 penalty (the section's own
     history: a raw-MSE objective picked only the lowest widths); at scale 1 the
     penalty still drowns the error's gradient within 500 steps; in percent
     the error term and the penalty pull with comparable force while the
     relaxed budget still holds to about 1e-2 bit.
R10  "PD" is primal-dual, with one step size: the tensor parameters take plain
     gradient-descent steps on the loss, the multiplier ascent steps
     lambda += step (bpw - target) from lambda = 0.5 (descending on it, as the
     pseudo-code writes it, leaves the loss unbounded below).  The section gives
     no rate; the step is 1/L, L = 2e4 ((b_max - b_min)/4)^2 sum_i w_i^2 the
     Lipschitz bound of the penalty's gradient (w_i = n_i / sum n), the largest
     step for which the stiff budget term cannot oscillate.
R11  Rounding keeps the budget (largest remainder): every tensor starts at the
     candidate at or below its continuous width; then, in order of the largest
     fraction of the way to the next candidate (earlier tensor first on ties),
     a tensor moves up one candidate when the bits it adds still fit in
     target * sum n.  The kept restart has the lowest exact objective among
     those within the budget; if none is, the lowest bpw.  Ties go to the
     earlier restart.  (The section's own allocation lands 0.05 bit over its
     5.0 target, which rounding to the nearest width would also do.)
R12  The restarts' starting parameters (0.5 * standard normal per tensor in
     the section) are an input, so that every implementation sees the same
     draws.
"""
from __future__ import annotations

import numpy as np

from .ddg_oracle import dequant_f32, quantize_groups

__all__ = ["PD_CANDIDATES", "quant_sse_rows", "sse_table", "mse_table", "pd_objective", "pd_loss_grad",
           "pd_search", "pd_exhaustive", "round_to_budget", "pd_step"]

PD_CANDIDATES = (3, 4, 5, 6, 7)
PENALTY = 1.0e4          # the section's quadratic budget penalty
ERROR_PERCENT = 100.0    # R9: the error term in percent of the uniform allocation's


def quant_sse_rows(w, bits: int) -> np.ndarray:
    """Per-row sum over the row of (w - w_hat32)^2 in float64, w_hat32 the
    float32 dequantized weight of the §3.1 quantizer at `bits`."""
    w = np.asarray(w, dtype=np.float32)
    q_u, s = quantize_groups(w, bits)
    w_hat = dequant_f32(q_u, s, bits)
    d = w.astype(np.float64) - w_hat.astype(np.float64)
    return np.sum(d * d, axis=1)


def sse_table(weights, candidates=PD_CANDIDATES):
    """(sse N x C, nparams N): the §3.2 objective's ||W_i - Q_c(W_i)||_F^2 of
    every tensor at every width, and each tensor's element count."""
    sse = np.empty((len(weights), len(candidates)), dtype=np.float64)
    n = np.empty(len(weights), dtype=np.int64)
    for i, w in enumerate(weights):
        n[i] = np.asarray(w).size
        for j, b in enumerate(candidates):
            sse[i, j] = quant_sse_rows(w, b).sum()
    return sse, n


def mse_table(weights, candidates=PD_CANDIDATES):
    """(mse N x C, nparams N): per-weight MSE of every tensor at every width,
    the squared-error sum over the element count."""
    sse, n = sse_table(weights, candidates)
    return sse / n[:, None].astype(np.float64), n


def pd_objective(mse, nparams, bits, candidates=PD_CANDIDATES):
    """(parameter-weighted MSE, bits per weight) of a discrete allocation."""
    mse = np.asarray(mse, dtype=np.float64)
    n = np.asarray(nparams, dtype=np.float64)
    idx = np.array([list(candidates).index(int(b)) for b in bits])
    tot = n.sum()
    e = float(np.sum(n * mse[np.arange(len(n)), idx]) / tot)
    p = float(np.sum(n * np.asarray(bits, dtype=np.float64)) / tot)
    return e, p


def round_to_budget(bcont, nparams, target_bpw: float, candidates=PD_CANDIDATES):
    """R11: largest-remainder rounding of continuous widths onto the
    candidates within the budget target * sum n.  Returns the widths."""
    cand = np.asarray(candidates, dtype=np.float64)
    n = np.asarray(nparams, dtype=np.float64)
    b = np.asarray(bcont, dtype=np.float64)
    j = np.array([int(np.sum(cand <= x)) - 1 for x in b])     # candidate at or below
    j = np.clip(j, 0, len(cand) - 1)
    frac = np.zeros(len(b))
    up = j < len(cand) - 1
    frac[up] = (b[up] - cand[j[up]]) / (cand[j[up] + 1] - cand[j[up]])
    budget = target_bpw * float(np.sum(n))
    spent = float(np.sum(n * cand[j]))
    for i in sorted(range(len(b)), key=lambda i: (-frac[i], i)):
        if frac[i] > 0.0:
            add = n[i] * (cand[j[i] + 1] - cand[j[i]])
            if spent + add <= budget:
                j[i] += 1
                spent += add
    return cand[j].astype(np.int64)


def pd_step(nparams, candidates=PD_CANDIDATES) -> float:
    """R10: 1 / L, L = 2 * penalty * ((b_max - b_min) / 4)^2 * sum_i w_i^2."""
    n = np.asarray(nparams, dtype=np.float64)
    w = n / n.sum()
    span = (max(candidates) - min(candidates)) / 4.0
    return 1.0 / (2.0 * PENALTY * span * span * float(np.sum(w * w)))


def pd_loss_grad(t, lam, m, wgt, cand, target_bpw: float, temp: float):
    """The relaxed loss of §3.2 and its gradient with respect to the tensor
    parameters t: error(t) + lam (bpw - target) + 1e4 (bpw - target)^2, where
    error = sum_i wgt_i sum_c softmax_c(-|b_i - c| / temp) m_ic and
    b_i = bmin + sigmoid(t_i) (bmax - bmin).  Returns (loss, grad, bpw)."""
    bmin, bmax = cand.min(), cand.max()
    u = 1.0 / (1.0 + np.exp(-t))
    b = bmin + u * (bmax - bmin)
    a = -np.abs(b[:, None] - cand[None, :]) / temp
    a = a - a.max(axis=1, keepdims=True)
    e = np.exp(a)
    sw = e / e.sum(axis=1, keepdims=True)
    s = np.sum(sw * m, axis=1)
    bpw = float(np.sum(wgt * b))
    gap = bpw - target_bpw
    loss = float(np.sum(wgt * s)) + lam * gap + PENALTY * gap * gap
    ds_db = np.sum(sw * (m - s[:, None]) * (-np.sign(b[:, None] - cand[None, :]) / temp), axis=1)
    dl_db = wgt * (ds_db + lam + 2.0 * PENALTY * gap)
    return loss, dl_db * (bmax - bmin) * u * (1.0 - u), bpw


def pd_search(mse, nparams, target_bpw: float, t_init, iters: int = 500,
              candidates=PD_CANDIDATES, trace=None):
    """The §3.2 search (readings R7-R12).  t_init: restarts x N starting
    parameters.  Returns dict(bits, mse, bpw, restart).  When `trace` is a
    list, one dict per (restart, iteration) is appended to it: the restart,
    the iteration, the temperature it used, and t and lambda after its update."""
    mse = np.asarray(mse, dtype=np.float64)
    n = np.asarray(nparams, dtype=np.float64)
    cand = np.asarray(candidates, dtype=np.float64)
    bmin, bmax = cand.min(), cand.max()
    wgt = n / n.sum()
    # R9: in percent of the uniform allocation at the candidate nearest the target
    j0 = int(np.argmin(np.abs(cand - target_bpw)))
    ref = float(np.sum(wgt * mse[:, j0]))
    m = ERROR_PERCENT * mse / ref if ref > 0 else ERROR_PERCENT * mse
    step = pd_step(n, candidates)                                # R10
    best = None
    for r, t0 in enumerate(np.asarray(t_init, dtype=np.float64)):
        t = t0.copy()
        lam = 0.5
        for it in range(iters):
            temp = max(2.0 * (1.0 - it / iters), 0.05)
            _, g, bpw = pd_loss_grad(t, lam, m, wgt, cand, target_bpw, temp)
            t = t - step * g
            lam = lam + step * (bpw - target_bpw)
            if trace is not None:
                trace.append({"restart": r, "it": it, "temp": temp, "t": t.copy(), "lam": lam})
        u = 1.0 / (1.0 + np.exp(-t))
        bits = round_to_budget(bmin + u * (bmax - bmin), n, target_bpw, candidates)   # R11
        e_r, p_r = pd_objective(mse, n, bits, candidates)
        key = (0, e_r, p_r) if p_r <= target_bpw + 1e-9 else (1, p_r, e_r)
        if best is None or key < best[0]:
            best = (key, bits.astype(np.int64), e_r, p_r, r)
    return {"bits": best[1], "mse": best[2], "bpw": best[3], "restart": best[4]}


def pd_exhaustive(mse, nparams, target_bpw: float, candidates=PD_CANDIDATES):
    """Brute force over every allocation (tiny N only): the lowest objective
    within the budget.  Returns (bits, mse, bpw)."""
    import itertools
    best = None
    for combo in itertools.product(candidates, repeat=len(nparams)):
        e, p = pd_objective(mse, nparams, combo, candidates)
        if p <= target_bpw + 1e-9 and (best is None or (e, p) < best[1:]):
            best = (np.array(combo, dtype=np.int64), e, p)
    return best
