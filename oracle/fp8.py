"""Plain fp64 CPU oracle for the FP8 forward with incoherent processing.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH. Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
or call this module. It shares no code with the HIP library.

What the method does (deepfa.ir page, section "پردازش ناهمدوس برای FP8"
under FlashAttention 3; unite.ai page, section on FlashAttention-3, items 2
and 3): the scores Q K^T are formed from FP8 operands, and before they are
quantised Q and K are multiplied by a Hadamard transform with random signs,
which spreads outlier channels over all channels and lowers the
quantisation error. The pages give no more than that; the readings used:

* The transform is M = diag(s) H with s in {-1, +1}^d the random signs (an
  input: drawn once per call by the caller) and H the d x d Sylvester
  Hadamard matrix (entries +-1, H H^T = d I). Then (Q M)(K M)^T = d Q K^T.
* FP8 is OCP e4m3 (4 exponent bits, bias 7, 3 mantissa bits, subnormals,
  largest finite value 448), rounded to nearest, ties to even, saturating at
  +-448.
* Scales are powers of two so that scaling is exact: each query row i gets
  a_i = 2^ceil(log2(max_c |Q~_ic| / 448)) and each tile t of 64 consecutive
  keys b_t = 2^ceil(log2(max |K~_jc| / 448)) over the tile (1 when the
  maximum is 0); q8 = e4m3(Q~ / a), k8 = e4m3(K~ / b).
* S_ij = scale / d * a_i * b_t(j) * sum_c q8_ic k8_jc; the mask and lse
  follow the exact definition (``oracle.attention``) on these scores.
* The second product is FP8 too. V is quantised without a rotation, with a
  power-of-two scale per column and block of 32 consecutive keys
  (v8 = e4m3(V / s), same scale rule). The probabilities are taken relative
  to the row maximum rounded up to a whole power of two,
  P_ij = 2^(log2(e) S_ij - m_i) with m_i = ceil(log2(e) max_j S_ij), so that
  P is in (0, 1] and any power-of-two change of reference rescales P
  exactly. P is rounded with the power-of-two scale the rule above gives its
  bound 1, 2^-8 (codes e4m3(2^8 P), so the largest probabilities sit at the
  top of the e4m3 range and subnormals only start below 2^-14), and the row
  sum uses the unrounded P: O_i = sum_j 2^-8 e4m3(2^8 P_ij) s_jc v8_jc / sum_j P_ij.
* Plain FP8 (no incoherent processing, the pages' baseline) is the same with
  M = I, so S_ij = scale * a_i b_t(j) sum_c q8_ic k8_jc.
"""

from __future__ import annotations

import numpy as np

from . import attention as _att

E4M3_MAX = 448.0
KEY_TILE = 64   # keys sharing one K scale
V_BLOCK = 32    # consecutive keys sharing one V scale per column


def e4m3_round(x):
    """Round to the nearest OCP e4m3 value, ties to even, saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # exponent e of each value's binade [2^e, 2^(e+1)) (frexp: a = f 2^k,
    # f in [0.5, 1)), at least -6: the subnormals share the step 2^-9 of the
    # lowest normal binade
    _, k = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(k - 1.0, -6.0)
    step = np.exp2(e - 3.0)  # 3 mantissa bits
    q = np.round(a / step) * step  # numpy rounds half to even
    q = np.minimum(q, E4M3_MAX)
    return np.where(x < 0, -q, q)


def e4m3_values():
    """Every finite non-negative e4m3 value, ascending."""
    vals = [m / 8.0 * 2.0 ** -6 for m in range(8)]  # zero and subnormals
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue  # NaN
            vals.append((1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


def hadamard(d):
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def pow2_scale(maxabs):
    """2^ceil(log2(maxabs / 448)), and 1 where maxabs is 0."""
    maxabs = np.asarray(maxabs, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(maxabs > 0, maxabs, E4M3_MAX) / E4M3_MAX))
    return np.exp2(e)


def quantize_rows(x):
    """(codes, scales): each row of x scaled by its power-of-two scale."""
    a = pow2_scale(np.max(np.abs(x), axis=1))
    return e4m3_round(x / a[:, None]), a


def quantize_tiles(x, tile=KEY_TILE):
    """(codes, per-row scales): rows in tiles of `tile` share one scale."""
    n = x.shape[0]
    a = np.empty(n)
    for t0 in range(0, n, tile):
        a[t0:t0 + tile] = pow2_scale(np.max(np.abs(x[t0:t0 + tile])))
    return e4m3_round(x / a[:, None]), a


def quantize_key_blocks(x, block=V_BLOCK):
    """(codes, per-element scales): in every column, each run of `block`
    consecutive rows shares one scale."""
    n = x.shape[0]
    a = np.empty(x.shape)
    for r0 in range(0, n, block):
        a[r0:r0 + block] = pow2_scale(np.max(np.abs(x[r0:r0 + block]), axis=0))[None, :]
    return e4m3_round(x / a), a


def fp8_scores(q, k, scale, signs=None, quantize=True):
    """Scaled scores S (N x N) of one head from FP8 operands. signs: the d
    random signs of the incoherent processing, or None for plain FP8.
    quantize=False keeps the transformed operands exact (rotation only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[1]
    if signs is not None:
        m = np.asarray(signs, dtype=np.float64)[:, None] * hadamard(d)
        q, k, rescale = q @ m, k @ m, 1.0 / d
    else:
        rescale = 1.0
    if quantize:
        q8, a = quantize_rows(q)
        k8, b = quantize_tiles(k)
        return scale * rescale * (a[:, None] * (q8 @ k8.T) * b[None, :])
    return scale * rescale * (q @ k.T)


def forward_fp8_head(q, k, v, scale, causal, signs=None, quantize=True):
    """(O, lse) of one head: the FP8 scores of ``fp8_scores`` under the mask
    of ``oracle.attention``, then O = e4m3(P) V~ / rowsum(P) with
    P = 2^(log2(e) S - m), m the row maximum of log2(e) S rounded up to an
    integer, and V~ the block-quantised V. quantize=False keeps every operand
    exact (O is then the exact attention output)."""
    s = fp8_scores(q, k, scale, signs, quantize)
    n = s.shape[0]
    left, right = _att.window_bounds(causal)
    keys = np.arange(n)[None, :]
    rows = np.arange(n)[:, None]
    if left >= 0:
        s = np.where(keys >= rows - left, s, -np.inf)
    if right >= 0:
        s = np.where(keys <= rows + right, s, -np.inf)
    lse = _att._row_softmax_stats(s)
    v = np.asarray(v, dtype=np.float64)
    if not quantize:
        return np.exp(s - lse[:, None]) @ v, lse
    m = np.ceil(np.max(s, axis=1, keepdims=True) / np.log(2.0))
    p = np.exp2(s / np.log(2.0) - m)
    v8, vs = quantize_key_blocks(v)
    ps = pow2_scale(1.0)
    return (ps * e4m3_round(p / ps) @ (v8 * vs)) / np.sum(p, axis=1, keepdims=True), lse
