"""Error of the FP8 forward against EXACT attention, bounded from the e4m3
unit roundoff alone: the parity of record of the FP8 path, independent of
how any kernel (or the FP8 oracle) organises its quantisation.

The method (deepfa.ir page, FlashAttention 3, section on incoherent
processing for FP8) forms Q K^T from FP8 operands after a random-sign
Hadamard rotation of Q and K, and P V from FP8 operands. Every e4m3 rounding
of a value x, on any power-of-two scale s for which x / s stays in range,
errs by at most u |x| (u = 2^-4: three mantissa bits, nearest rounding)
when x / s is normal, and by half a subnormal step, 2^-10 s, otherwise.
Modelling each rounding as an independent error, zero-mean and uniform on
+-(that half step), its variance is at most h^2 / 3 with h = max(u |x|,
2^-10 s). To first order in these errors the output of query row i,
column c, moves by

  dO_ic = sum_j P_ij (V_jc - O_ic) dS_ij + sum_j P_ij V_jc (psi_jc + rho_ij)

with dS_ij = c0 sum_m (q~_im k~_jm)(theta_im + phi_jm) the score error
(c0 = scale / d when rotated, scale otherwise; q~, k~ the rotated, exact
operands), theta, phi, psi, rho the relative roundings of q~, k~, V and P.
Its variance sigma_ic^2 is the sum of:
  theta: c0^2 sum_m var(dq~_im) G_icm^2,
         G_icm = sum_j P_ij (V_jc - O_ic) k~_jm
  phi:   c0^2 sum_j P_ij^2 (V_jc - O_ic)^2 sum_m q~_im^2 var(dk~_jm)
  psi:   sum_j P_ij^2 var(dV_jc)
  rho:   sum_j var(dP_ij) V_jc^2
with var(dx) the variance bound of the rounding of x (absolute),
all computed here in fp64 from the exact inputs. The scales s entering the
subnormal floors are taken at their largest possible values for any choice
of the sets that share a scale (a set's maximum is at most the head's):
2^ceil(log2(max/448)) of the whole row (Q), of the whole head (K), of each
column of the head (V), and 2^-6 for probabilities (largest 1).

The expansion is first order in the score errors, so it is used only where
they are small: the check first requires the score error's standard
deviation, sqrt(var(dS_ij)), to stay below SCORE_SD_MAX for every pair. Inputs
with strong outlier channels in plain FP8 (scores off by O(1)) are outside
that range; there the method-level claim (incoherent processing lowers the
error) has its own test.

Gate per element: |O - O_exact| <= KAPPA sigma + 2^-8 |O_exact| + TAU, with
2^-8 |O| the bf16 rounding of the output, TAU covering fp32 accumulation and
the second-order terms; and over a head, the relative L2 error at most
L2_FACTOR times the model's root-mean-square prediction plus that of the
output rounding. KAPPA, L2_FACTOR and TAU are checked on the CPU against the
fp64 FP8 oracle (test_fp8_exact_bound_holds_for_the_oracle): the largest
ratio |error| / sigma it reaches on these inputs is recorded there.
"""

from __future__ import annotations

import numpy as np

import oracle

U = 2.0 ** -4          # e4m3 unit roundoff (normal values)
BF16_U = 2.0 ** -8     # bf16 rounding of the output
KAPPA = 7.0
TAU = 2e-5
L2_FACTOR = 1.25
SCORE_SD_MAX = 0.15


def _pow2_scale(maxabs):
    maxabs = np.asarray(maxabs, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(maxabs > 0, maxabs, 448.0) / 448.0))
    return np.exp2(e)


def _var(x, scale):
    """Variance bound of one e4m3 rounding of x on a grid of scale `scale`."""
    h = np.maximum(U * np.abs(x), 2.0 ** -10 * scale)
    return h * h / 3.0


def fp8_error_sd(q, k, v, scale, causal, signs, rows=None):
    """sigma (first-order standard deviation of the FP8 output's error) for
    query rows `rows` (all by default) of one head: [len(rows), d]."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n, d = q.shape
    if signs is None:
        qt, kt, c0 = q, k, scale
    else:
        m = np.asarray(signs, dtype=np.float64)[:, None] * oracle.hadamard(d)
        qt, kt, c0 = q @ m, k @ m, scale / d
    rows = np.arange(n) if rows is None else np.asarray(rows)
    p = oracle.probabilities_head(q, k, scale, causal)[rows]          # exact P
    o = p @ v
    var_q = _var(qt[rows], _pow2_scale(np.max(np.abs(qt[rows]), axis=1))[:, None])
    var_k = _var(kt, _pow2_scale(np.max(np.abs(kt))))
    var_v = _var(v, _pow2_scale(np.max(np.abs(v), axis=0))[None, :])
    score_sd = np.sqrt(c0 * c0 * (var_q @ (kt ** 2).T + (qt[rows] ** 2) @ var_k.T))
    if np.max(score_sd) > SCORE_SD_MAX:
        raise ValueError(f"score error sd {np.max(score_sd):.3f} above {SCORE_SD_MAX}: "
                         "outside the first-order model's range")
    p2 = p * p
    # theta: G_icm = sum_j P_ij V_jc k~_jm - O_ic sum_j P_ij k~_jm
    t = (p @ (v[:, :, None] * kt[:, None, :]).reshape(n, d * d)).reshape(len(rows), d, d)
    g = t - o[:, :, None] * (p @ kt)[:, None, :]
    s_theta = c0 * c0 * np.einsum("im,icm->ic", var_q, g * g)
    # phi: sum_j P_ij^2 (V_jc - O_ic)^2 w_ij, w_ij = sum_m q~_im^2 var(phi_jm)
    w = p2 * ((qt[rows] ** 2) @ var_k.T)
    s_phi = c0 * c0 * (w @ (v * v) - 2.0 * o * (w @ v) + o * o * w.sum(axis=1, keepdims=True))
    # psi (V) and rho (P, relative to the row's reference: var <= (u P)^2/3 + floor)
    s_psi = p2 @ var_v
    var_rho = np.maximum(U * p, 2.0 ** -10 * 2.0 ** -6) ** 2 / 3.0
    s_rho = var_rho @ (v * v)
    return np.sqrt(np.maximum(s_theta + s_phi + s_psi + s_rho, 0.0))


def check_fp8_vs_exact(o, q, k, v, scale, causal, signs, what, rows=None, log=print):
    """The FP8 output o (rows `rows` of one head, as float) against exact
    attention with the bound above. Returns (worst |err| / sigma, rel L2)."""
    o = np.asarray(o, dtype=np.float64)
    n = np.shape(q)[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    exact, _ = oracle.forward_head(q, k, v, scale, causal, rows=rows)
    sd = fp8_error_sd(q, k, v, scale, causal, signs, rows)
    err = np.abs(o - exact)
    bound = KAPPA * sd + BF16_U * np.abs(exact) + TAU
    ratio = float(np.max(err / np.maximum(sd, 1e-30)))
    rel = float(np.linalg.norm(o - exact) / np.linalg.norm(exact))
    predicted = float(np.sqrt(np.sum(sd ** 2) + np.sum((BF16_U / np.sqrt(3) * exact) ** 2))
                      / np.linalg.norm(exact))
    log(f"  {what}: FP8 vs exact: rel L2 {rel:.4f} (model {predicted:.4f}), "
        f"worst |err|/sigma {ratio:.2f}, worst bound use {float(np.max(err / bound)):.3f}")
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert np.all(err <= bound), (what, ratio)
    assert rel <= L2_FACTOR * predicted, (what, rel, predicted)
    return ratio, rel
