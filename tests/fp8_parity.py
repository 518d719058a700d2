"""Check of the FP8 kernel against its own quantisation design
(oracle.forward_fp8_head follows that design: per-row Q scales, 64-key-tile
K scales, 32-key V blocks, P relative to a power-of-two reference and
rounded with the scale 2^-8). This is not the parity of record, which is
the kernel-independent bound against exact attention in fp8_exact_bound.py.

Both sides round the same values onto the same e4m3 grids, so their results
are identical except where a value lies so close to a rounding midpoint that
the GPU's fp32 arithmetic and the oracle's fp64 arithmetic can pick the two
different neighbours; both are then correct. This check computes, from the
oracle alone, which decisions are ambiguous and how far each may move O, and
requires the GPU output to lie within that allowance of the oracle's:

* rotated Q and K codes whose value (in units of its scale) lies within
  1e-5 of its row's largest magnitude of a midpoint (the GPU rotates in
  fp32: at most 7 butterfly roundings of sums bounded by sqrt(d) times the
  row's largest value, 2^-24 each, about 5e-6); a flip moves the code one
  grid step and the scores of the row (Q) or key (K) by at most
  scale * a * b * step * |other operand's code| (/ d when rotated);
* probabilities 2^8 P within 2e-4 (relative), plus the score shifts above, of
  a midpoint (the GPU's scores are fp32 sums of up to d exact products,
  error at most about d 2^-24 sum|terms|, 1e-4 in the exponent for N(0,1)
  rows at d = 128, plus 1e-6 from exp2 and the fused multiply-add); a flip
  moves 2^-8 e4m3(2^8 P) by one grid step;
* a score shift dS changes P by at most P (e^dS - 1), the numerator and the
  row sum alike.

Bound per element: |O - O_ref| <= 2^-8 |O_ref| (bf16 output rounding) +
sum_j (flip_ij + 2 dP_ij) |V~_jc| / l_i + 1e-3 (fp32 accumulation), with
relative L2 error <= 5e-3 over the head as for the bf16 forward, counted on
what the ambiguous decisions do not explain: per element, the error less its
allowance for flips and score shifts (the flip_ij and dP_ij terms). Either
neighbour of an ambiguous midpoint is a correct rounding, and one flip of a
row's dominant probability moves that row by one e4m3 step of P (1/16 of
2^8 P in [128, 256)), which on a head of a few dozen rows alone exceeds 5e-3.
"""

from __future__ import annotations

import numpy as np

import oracle
from parity import O_REL_L2, log, metrics

GRID = oracle.e4m3_values()


def _neighbours(y):
    """Grid values around |y| (y within the e4m3 range): lo <= |y| <= hi."""
    a = np.abs(y)
    idx = np.clip(np.searchsorted(GRID, a, side="right") - 1, 0, len(GRID) - 1)
    lo = GRID[idx]
    hi = GRID[np.minimum(idx + 1, len(GRID) - 1)]
    return a, lo, hi


def _ambiguous_codes(x, window):
    """Codes whose value x (already divided by its scale) lies within `window`
    times the row's largest |x| of a rounding midpoint; returns (mask, step)."""
    a, lo, hi = _neighbours(x)
    near = np.abs(a - (lo + hi) / 2) <= window * np.max(a, axis=-1, keepdims=True)
    return near & (hi > lo), hi - lo


def fp8_allowance(q, k, v, scale, causal, signs):
    """(O_ref, lse_ref, bound, n_flip_candidates) for one head."""
    d = q.shape[1]
    ro, rl = oracle.forward_fp8_head(q, k, v, scale, causal, signs)
    if signs is None:
        qt, kt, rescale = q, k, 1.0
    else:
        m = np.asarray(signs, dtype=np.float64)[:, None] * oracle.hadamard(d)
        qt, kt, rescale = q @ m, k @ m, 1.0 / d
    q8, a = oracle.quantize_rows(qt)
    k8, b = oracle.quantize_tiles(kt)
    ds = np.zeros((q.shape[0], k.shape[0]))
    if signs is not None:
        amb_q, step_q = _ambiguous_codes(qt / a[:, None], 1e-5)
        amb_k, step_k = _ambiguous_codes(kt / b[:, None], 1e-5)
        ds = np.abs(scale) * rescale * a[:, None] * b[None, :] * (
            (amb_q * step_q) @ np.abs(k8).T + np.abs(q8) @ (amb_k * step_k).T)
    s = oracle.fp8_scores(q, k, scale, signs)
    n = s.shape[0]
    left, right = oracle.window_bounds(causal)
    keys, rows = np.arange(n)[None, :], np.arange(n)[:, None]
    vis = np.ones((n, n), dtype=bool)
    if left >= 0:
        vis &= keys >= rows - left
    if right >= 0:
        vis &= keys <= rows + right
    s = np.where(vis, s, -np.inf)
    mref = np.ceil(np.max(s, axis=1, keepdims=True) / np.log(2.0))
    p = np.exp2(s / np.log(2.0) - mref)
    l = p.sum(axis=1, keepdims=True)
    y = 256.0 * p
    ay, lo, hi = _neighbours(y)
    window = y * (2e-4 + np.expm1(ds))
    flip = (np.abs(ay - (lo + hi) / 2) <= window) & (hi > lo) & vis
    v8, vs = oracle.quantize_key_blocks(v)
    av = np.abs(v8 * vs)
    dp = p * np.expm1(ds)
    extra = ((flip * (hi - lo) / 256.0 + 2.0 * dp) @ av) / l
    bound = 2.0 ** -8 * np.abs(ro) + extra + 1e-3
    return ro, rl, bound, extra, int(flip.sum())


def check_fp8_o(o, q, k, v, scale, causal, signs, what):
    """O of the FP8 path against the oracle with the allowance above; returns lse_ref."""
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    ro, rl, bound, ambiguous, flips = fp8_allowance(q, k, v, scale, causal, signs)
    o = np.asarray(o, dtype=np.float64)
    excess = float(np.max(np.abs(o - ro) - bound))
    max_abs, rel = metrics(o, ro)
    # the relative L2 of what the ambiguous decisions do not explain
    rest = np.maximum(np.abs(o - ro) - ambiguous, 0.0)
    denom = float(np.linalg.norm(ro))
    rel_rest = float(np.linalg.norm(rest)) / denom if denom > 0 else float(np.linalg.norm(rest))
    log(f"  {what}: O max_abs={max_abs:.3e} rel_l2={rel:.3e} (without ambiguous decisions "
        f"{rel_rest:.3e}) ambiguous P={flips} worst bound margin={-excess:.3e}")
    assert excess <= 0.0 and rel_rest <= O_REL_L2, (what, max_abs, rel, rel_rest, excess)
    return rl
