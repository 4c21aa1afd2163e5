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

Readings where the section is silent (each is repeated in the design doc):

R7   Candidate widths are the packable ones, 3..7; b_min = 3, b_max = 7.
R8   dist(b, c) = |b - c|; the soft weights are softmax_c(-|b - c| / temp),
     temp = max(2 (1 - it / iters), 0.05).
R9   The error table enters normalised: per-weight MSE of tensor i at width
     c, divided by the parameter-weighted MSE of the uniform allocation at the
     candidate nearest the target.  Raw per-weight MSEs (~1e-7 for DiT
     weights) would vanish next to the 1e4 penalty, and the section's own
     history (a raw-MSE objective that picked only the lowest widths) is
     consistent with that.
R10  "PD" is primal-dual: the tensor parameters take Adam steps on the loss
     (lr 0.05, beta 0.9 / 0.999, eps 1e-8; the section names plain gradient
     descent without a rate), the multiplier takes ascent steps
     lambda += lr_dual (bpw - target) from lambda = 0.5.  Descending on the
     multiplier, as the pseudo-code writes it, leaves the loss unbounded.
R11  Rounding: each tensor takes the candidate nearest its continuous width
     (ties to the lower width).  The kept restart has the lowest exact
     objective among those within the budget (bpw <= target + 1e-9); if none
     is, the lowest bpw.  Ties go to the earlier restart.
R12  The restarts' starting parameters (0.5 * standard normal per tensor in
     the section) are an input, so that every implementation sees the same
     draws.
"""
from __future__ import annotations

import numpy as np

from .ddg_oracle import dequant_f32, quantize_groups

__all__ = ["PD_CANDIDATES", "quant_sse_rows", "mse_table", "pd_objective", "pd_loss_grad",
           "pd_search", "pd_exhaustive"]

PD_CANDIDATES = (3, 4, 5, 6, 7)
PENALTY = 1.0e4          # the section's quadratic budget penalty


def quant_sse_rows(w, bits: int) -> np.ndarray:
    """Per-row sum over the row of (w - w_hat32)^2 in float64, w_hat32 the
    float32 dequantized weight of the §3.1 quantizer at `bits`."""
    w = np.asarray(w, dtype=np.float32)
    q_u, s = quantize_groups(w, bits)
    w_hat = dequant_f32(q_u, s, bits)
    d = w.astype(np.float64) - w_hat.astype(np.float64)
    return np.sum(d * d, axis=1)


def mse_table(weights, candidates=PD_CANDIDATES):
    """(mse N x C, nparams N): per-weight MSE of every tensor at every width."""
    mse = np.empty((len(weights), len(candidates)), dtype=np.float64)
    n = np.empty(len(weights), dtype=np.int64)
    for i, w in enumerate(weights):
        n[i] = np.asarray(w).size
        for j, b in enumerate(candidates):
            mse[i, j] = quant_sse_rows(w, b).sum() / n[i]
    return mse, n


def pd_objective(mse, nparams, bits, candidates=PD_CANDIDATES):
    """(parameter-weighted MSE, bits per weight) of a discrete allocation."""
    mse = np.asarray(mse, dtype=np.float64)
    n = np.asarray(nparams, dtype=np.float64)
    idx = np.array([list(candidates).index(int(b)) for b in bits])
    tot = n.sum()
    e = float(np.sum(n * mse[np.arange(len(n)), idx]) / tot)
    p = float(np.sum(n * np.asarray(bits, dtype=np.float64)) / tot)
    return e, p


def _nearest(bcont, cand):
    """Candidate nearest each continuous width, ties to the lower one (R11)."""
    d = np.abs(bcont[:, None] - cand[None, :])
    return cand[np.argmin(d, axis=1)]        # argmin takes the first (lower) on ties


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
              candidates=PD_CANDIDATES, lr: float = 0.05, lr_dual: float = 0.05):
    """The §3.2 search (readings R7-R12).  t_init: restarts x N starting
    parameters.  Returns dict(bits, mse, bpw, restart)."""
    mse = np.asarray(mse, dtype=np.float64)
    n = np.asarray(nparams, dtype=np.float64)
    cand = np.asarray(candidates, dtype=np.float64)
    bmin, bmax = cand.min(), cand.max()
    tot = n.sum()
    wgt = n / tot
    # R9: normalise by the uniform allocation at the candidate nearest the target
    j0 = int(np.argmin(np.abs(cand - target_bpw)))
    ref = float(np.sum(wgt * mse[:, j0]))
    m = mse / ref if ref > 0 else mse
    best = None
    for r, t0 in enumerate(np.asarray(t_init, dtype=np.float64)):
        t = t0.copy()
        lam = 0.5
        m1 = np.zeros_like(t)
        m2 = np.zeros_like(t)
        for it in range(iters):
            temp = max(2.0 * (1.0 - it / iters), 0.05)
            _, g, bpw = pd_loss_grad(t, lam, m, wgt, cand, target_bpw, temp)
            gap = bpw - target_bpw
            # Adam step on t (R10)
            m1 = 0.9 * m1 + 0.1 * g
            m2 = 0.999 * m2 + 0.001 * g * g
            mh = m1 / (1.0 - 0.9 ** (it + 1))
            vh = m2 / (1.0 - 0.999 ** (it + 1))
            t = t - lr * mh / (np.sqrt(vh) + 1e-8)
            lam = lam + lr_dual * gap                           # dual ascent (R10)
        u = 1.0 / (1.0 + np.exp(-t))
        bits = _nearest(bmin + u * (bmax - bmin), cand)
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
