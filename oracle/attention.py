"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call this module. It shares no code with the HIP library: it takes
numpy fp64 arrays and uses numpy matmul, exp, log and max as its only
primitives, in the order the definition states them.

What it computes (per batch b and head h, all heads independent):

* Attention(Q, K, V) = softmax(Q K^T * scale) V, the formula of the Persian
  page "Flash Attention: بهینه‌سازی مکانیزم توجه در ترنسفورمرها" (deepfa.ir),
  section "ساختار مکانیزم توجه", and the ``standard_attention`` example of
  the Italian page "Flash Attention: Rivoluzionando l'Efficienza dei Modelli
  Transformer" (unite.ai), introduction. The pages fix scale = 1/sqrt(d);
  here it is an argument (callers pass 1/sqrt(d)).
* The softmax is taken in its decomposed, max-subtracted form
  exp(x - m) / sum exp(x - m), m = max x: unite.ai page, section
  "La Matematica dietro Flash Attention", formula 1.
* Causal masking (keys j <= query i visible) is named but never defined on the
  pages; the plainest reading, the lower-triangular mask with equal query and
  key lengths, is used.
* Local (sliding-window) attention is named on the pages only as a coming
  variant (nearauto.com page, section "今後の仕事"; aiunderstanding.org page,
  section "Il futuro dell'attenzione flash"). The reading used generalises
  the causal mask: every function's ``causal`` argument may also be a pair
  (left, right), key j visible to query i iff i - left <= j <= i + right, a
  bound of -1 meaning none on that side; True is (-1, 0), False (-1, -1).
* Block-sparse attention is likewise named on the pages only as a coming
  variant (nearauto.com page, section "今後の仕事": block-sparse attention)
  and defined nowhere. The reading used: a mask over blocks of MASK_BLOCK
  query rows x MASK_BLOCK keys of the score matrix; the scores of a block
  the mask marks 0 are treated as masked keys (-inf), on top of the
  causal or window mask. A row left with no visible key has O = 0 and
  lse = -inf, and no gradient flows through it. Every function taking
  ``causal`` also takes ``block_mask``: None (no mask), a 2-D array of
  [ceil(N/MASK_BLOCK)] x [ceil(N/MASK_BLOCK)] entries (nonzero = computed),
  or, for ``forward`` and ``backward``, one such array per (batch, head).
* The per-row logsumexp lse_i = ln sum_j exp(scale * q_i . k_j) over visible
  keys is not on the pages; it is the row statistic the backward pass needs
  to recompute P without storing it (deepfa.ir page, section
  "تکنیک 2: محاسبه مجدد", recomputation). Natural log of the scaled scores.
* The backward pass is not on the pages; it is the calculus of the
  definition above: with P the softmax, D_i = sum_k dO_ik O_ik,
  dP = dO V^T, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q,
  dV = P^T dO.
* Grouped-query and multi-query attention (nearauto.com page, section
  "新機能"): several query heads share one K/V head. ``forward`` and
  ``backward`` take K and V with Hkv heads, Hkv dividing H; query head h
  reads K/V head h // (H / Hkv) (consecutive groups: the page does not say
  which heads form a set), and a shared K/V head's gradient is the sum over
  its query heads.
* ``merge`` combines the results over two disjoint key sets; the unite.ai
  page's formula 2 ("Unione della Softmax") is garbled as printed, and the
  reading used is the plain one: rescale each part's unnormalised sums by
  exp(m_part - m) with m the larger maximum, i.e. in lse form
  lse = ln(e^lse1 + e^lse2), O = e^(lse1-lse) O1 + e^(lse2-lse) O2.

Pins: tests/test_oracle_pins.py checks this module against closed forms,
textbook special cases, torch's fp64 CPU attention and autograd, finite
differences, brute-force loops and the fixtures under tests/golden/.
"""

from __future__ import annotations

import numpy as np

# Rows of the score matrix formed at once; each output row depends only on its
# own query row, so chunking rows changes nothing in the result.
_ROW_CHUNK = 512

# Query rows and keys per block of a block-sparse mask.
MASK_BLOCK = 128


def _check_head(q, k, v):
    if q.ndim != 2 or k.ndim != 2 or v.ndim != 2:
        raise ValueError("per-head arrays must be 2-D [N, d]")
    if k.shape != v.shape or q.shape[1] != k.shape[1]:
        raise ValueError("shape mismatch between q, k, v")


def window_bounds(causal):
    """(left, right) of a mask argument: key j is visible to query i iff
    (left < 0 or j >= i - left) and (right < 0 or j <= i + right).

    ``causal`` is False (every key), True (keys j <= i: (-1, 0)) or a pair
    (left, right) of integers >= -1 (a local / sliding-window mask; -1: no
    bound on that side)."""
    if causal is None or isinstance(causal, (bool, np.bool_)):
        return (-1, 0) if causal else (-1, -1)
    left, right = (int(x) for x in causal)
    if left < -1 or right < -1:
        raise ValueError(f"window bounds must be >= -1, got {causal}")
    return left, right


def _scores(q_rows, k, scale, row_ids, causal):
    """S = scale * Q K^T for the given query rows, masked keys set to -inf."""
    s = scale * (q_rows @ k.T)
    left, right = window_bounds(causal)
    keys = np.arange(k.shape[0])[None, :]
    rows = row_ids[:, None]
    if left >= 0:
        s = np.where(keys >= rows - left, s, -np.inf)
    if right >= 0:
        s = np.where(keys <= rows + right, s, -np.inf)
    return s


def _apply_block_mask(s, row_ids, block_mask):
    """Scores of the blocks a block-sparse mask marks 0 set to -inf."""
    if block_mask is None:
        return s
    bm = np.asarray(block_mask) != 0
    row_blocks = (np.asarray(row_ids) // MASK_BLOCK)[:, None]
    key_blocks = (np.arange(s.shape[1]) // MASK_BLOCK)[None, :]
    return np.where(bm[row_blocks, key_blocks], s, -np.inf)


def _head_mask(block_mask, b, h):
    """The block mask of head (b, h): None, one 2-D mask for every head, or
    a [B, H, ...] stack of them."""
    if block_mask is None:
        return None
    bm = np.asarray(block_mask)
    return bm if bm.ndim == 2 else bm[b, h]


def _row_softmax_stats(s):
    """Row max m and lse = m + ln sum exp(s - m) (decomposed softmax).

    A row with no visible key (cannot happen with Nq == Nk causal masks) gets
    lse = -inf and an all-zero probability row.
    """
    m = np.max(s, axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    total = np.sum(np.exp(s - m_safe[:, None]), axis=1)
    with np.errstate(divide="ignore"):
        lse = m_safe + np.log(total)
    lse = np.where(total > 0, lse, -np.inf)
    return lse


def forward_head(q, k, v, scale, causal, rows=None, block_mask=None):
    """Exact attention output and logsumexp for one head.

    q, k, v: float64 [N, d]. rows: optional 1-D array of query indices to
    compute (each row is independent of the others). block_mask: see the
    module docstring. Returns (O[rows], lse[rows]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check_head(q, k, v)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.zeros(rows.shape[0], dtype=np.float64)
    for start in range(0, rows.shape[0], _ROW_CHUNK):
        ids = rows[start:start + _ROW_CHUNK]
        s = _apply_block_mask(_scores(q[ids], k, scale, ids, causal), ids, block_mask)
        l_rows = _row_softmax_stats(s)
        with np.errstate(invalid="ignore"):
            p = np.exp(s - np.where(np.isfinite(l_rows), l_rows, 0.0)[:, None])
        p = np.where(np.isfinite(l_rows)[:, None], p, 0.0)
        out[start:start + ids.shape[0]] = p @ v
        lse[start:start + ids.shape[0]] = l_rows
    return out, lse


def probabilities_head(q, k, scale, causal, block_mask=None):
    """The full softmax matrix P (N x N) of one head; small N only. A row
    with no visible key (possible under a block mask) is all zeros."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    ids = np.arange(q.shape[0])
    s = _apply_block_mask(_scores(q, k, scale, ids, causal), ids, block_mask)
    lse = _row_softmax_stats(s)
    with np.errstate(invalid="ignore"):
        p = np.exp(s - lse[:, None])
    return np.where(np.isfinite(lse)[:, None], p, 0.0)


def backward_head(q, k, v, do, scale, causal, block_mask=None):
    """Gradients (dQ, dK, dV) of sum(dO * O) for one head, O = attention(q,k,v).

    Materialises the full N x N matrices. The forward output used for
    D_i = sum_k dO_ik O_ik is this oracle's own exact O.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _check_head(q, k, v)
    p = probabilities_head(q, k, scale, causal, block_mask)
    o = p @ v
    d_row = np.sum(do * o, axis=1)
    dp = do @ v.T
    ds = p * (dp - d_row[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    return dq, dk, dv


def kv_head(h, heads, kv_heads):
    """K/V head read by query head h when `heads` query heads share
    `kv_heads` K/V heads (grouped-query attention; kv_heads = 1 is
    multi-query attention, kv_heads = heads ordinary multi-head attention).

    The nearauto.com page, section "新機能", says each set of query heads
    shares one K/V head. It does not say which heads form a set; the reading
    used is consecutive groups of heads // kv_heads query heads."""
    if kv_heads < 1 or heads % kv_heads != 0:
        raise ValueError(f"{heads} query heads cannot share {kv_heads} K/V heads evenly")
    return h // (heads // kv_heads)


def forward(q, k, v, scale, causal, block_mask=None):
    """Batched forward: q [B, H, N, d], k and v [B, Hkv, N, d] float64 with
    Hkv dividing H (Hkv = H: multi-head) -> (O [B, H, N, d], lse [B, H, N]).
    Query head h attends over K/V head kv_head(h, H, Hkv); block_mask is per
    query head."""
    q = np.asarray(q, dtype=np.float64)
    bsz, heads, n, d = q.shape
    kv_heads = np.shape(k)[1]
    out = np.zeros((bsz, heads, n, v.shape[-1]), dtype=np.float64)
    lse = np.zeros((bsz, heads, n), dtype=np.float64)
    for b in range(bsz):
        for h in range(heads):
            g = kv_head(h, heads, kv_heads)
            out[b, h], lse[b, h] = forward_head(q[b, h], k[b, g], v[b, g], scale, causal,
                                                block_mask=_head_mask(block_mask, b, h))
    return out, lse


def backward(q, k, v, do, scale, causal, block_mask=None):
    """Batched backward over the shapes of ``forward`` -> (dQ, dK, dV). A K/V
    head read by several query heads receives the sum of their gradients (the
    chain rule for a shared input)."""
    q = np.asarray(q, dtype=np.float64)
    heads, kv_heads = q.shape[1], np.shape(k)[1]
    dq = np.zeros_like(q)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(q.shape[0]):
        for h in range(heads):
            g = kv_head(h, heads, kv_heads)
            dq[b, h], dk_h, dv_h = backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal,
                                                 block_mask=_head_mask(block_mask, b, h))
            dk[b, g] += dk_h
            dv[b, g] += dv_h
    return dq, dk, dv


def merge(o1, lse1, o2, lse2):
    """Combine attention over two disjoint key sets into attention over their union.

    Reading of the unite.ai page's "Unione della Softmax" formula: the part
    with the larger maximum is the reference and the other part's sums are
    rescaled by the exponential of the difference.
    """
    lse = np.logaddexp(lse1, lse2)
    w1 = np.exp(lse1 - lse)[..., None]
    w2 = np.exp(lse2 - lse)[..., None]
    return w1 * o1 + w2 * o2, lse
