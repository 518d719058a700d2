"""Shared helpers of the GPU parity tests: error metrics and tolerances.

Tolerances (HIP path vs the fp64 oracle on identical bf16 inputs):
  O          max abs error <= 1e-2 and relative L2 error <= 5e-3
  dQ, dK, dV relative L2 error <= 2e-2 over the head, and for every row r
             |g_r - ref_r| <= 3e-2 * max(|ref_r|, rms) (L2 norms of rows,
             rms = the root mean square row norm of the head's reference);
             a bf16 emulation of the backward arithmetic (P and dS rounded
             as MFMA operands, outputs rounded) gives worst rows of 4-5e-3
             at scale 1/sqrt(d) and 1.1e-2 at scale 0.4, while a zeroed row
             scores about 1 and a row missing one 64-key tile out of 16384
             about 6e-2. dQ rows get an additive allowance on top
             (dq_allowance): D_i is formed from the stored bf16 O, and
             dQ_i depends on D_i through -scale * sum_j P_ij K_j, which is
             large on short causal rows, whose dQ may itself be small
  lse        max abs error <= 1e-3 (lse never passes through bf16; the
             expected error is ~1e-5, set by fp32 sums and bf16 rounding of P)

These hold for the measured input distribution (N(0,1) inputs, scale
1/sqrt(d)), where the softmax rows are mild and the rounding errors of the
bf16 probabilities average out. Off that distribution (larger scales, scaled
queries: sharply peaked rows) O is checked element by element against the
bound the arithmetic gives: with u = 2^-8 the unit roundoff of bf16,
rounding each probability costs at most u * max_j |v_j| and rounding the
output at most u * |O|, so |O - O_ref| <= u * (|O_ref| + max_j |v_j|) + 1e-3
(the 1e-3 covers fp32 accumulation), still with the 5e-3 relative L2 gate.
The random sweep, which draws rows that see only a few keys, uses the tighter
form of that bound, with P |V| in place of max |v| (check_o_rounding).
"""

from __future__ import annotations

import sys

import numpy as np

import oracle

O_MAX_ABS = 1e-2
O_REL_L2 = 5e-3
GRAD_REL_L2 = 2e-2
GRAD_ROW_REL = 3e-2
LSE_MAX_ABS = 1e-3


def log(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def metrics(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if x.size == 0:
        return 0.0, 0.0
    diff = x - ref
    max_abs = float(np.max(np.abs(diff)))
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def check_o(o, ref, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    max_abs, rel = metrics(o, ref)
    log(f"  {what}: O max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= O_MAX_ABS and rel <= O_REL_L2, (what, max_abs, rel)


BF16_U = 2.0 ** -8


def check_o_peaked(o, ref, vmax, what):
    """Element-wise rounding bound for sharply peaked softmax rows."""
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    o = np.asarray(o, dtype=np.float64)
    bound = BF16_U * (np.abs(ref) + vmax) + 1e-3
    excess = float(np.max(np.abs(o - ref) - bound))
    max_abs, rel = metrics(o, ref)
    log(f"  {what}: O max_abs={max_abs:.3e} rel_l2={rel:.3e} worst bound margin={-excess:.3e}")
    assert excess <= 0.0 and rel <= O_REL_L2, (what, max_abs, rel, excess)


def check_o_rounding(o, ref, pav, what):
    """Element-wise bound of the forward's rounding, for O of one head.

    The kernels round each probability to bf16 for P.V (|error| <= u p_j)
    while l sums the unrounded ones, and round O to bf16 (<= u |O|), u = 2^-8;
    fp32 sums and exponentials add far below 1e-4 at these sizes. So
    |O_ik - O_ref_ik| <= u (|O_ref_ik| + sum_j P_ij |V_jk|) + 1e-4, with
    pav = P |V| from the oracle. On rows that average many keys this is about
    5e-3, tighter than the flat 1e-2; on rows that see a few keys with |O|
    above about 2.5 the output rounding alone exceeds 1e-2, which no bf16
    output can meet, and this bound is the gate there. The relative L2 gate
    of 5e-3 is kept."""
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    o = np.asarray(o, dtype=np.float64)
    bound = BF16_U * (np.abs(ref) + np.asarray(pav, dtype=np.float64)) + 1e-4
    excess = float(np.max(np.abs(o - ref) - bound)) if o.size else 0.0
    max_abs, rel = metrics(o, ref)
    log(f"  {what}: O max_abs={max_abs:.3e} rel_l2={rel:.3e} worst bound margin={-excess:.3e}")
    assert excess <= 0.0 and rel <= O_REL_L2, (what, max_abs, rel, excess)


def emulate_bf16_forward_head(q, k, v, scale, window, block_mask=None):
    """The forward's rounding design in fp64 for one head (test model, not
    the method): P = exp(S - max) over the visible keys, P.V with P rounded
    to bf16, divided by the unrounded row sum, O rounded to bf16. Rows with no
    visible key give 0."""
    import torch

    def bf16(x):
        return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()

    n = q.shape[0]
    s = (q @ k.T) * scale
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    wl, wr = window
    vis = np.ones((n, n), dtype=bool)
    if wl >= 0:
        vis &= j >= i - wl
    if wr >= 0:
        vis &= j <= i + wr
    if block_mask is not None:
        vis &= np.asarray(block_mask)[i // oracle.MASK_BLOCK, j // oracle.MASK_BLOCK] != 0
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - np.where(np.isfinite(m), m, 0.0))
    l = p.sum(axis=1, keepdims=True)
    return bf16((bf16(p) @ v) / np.where(l > 0, l, 1.0))


def check_lse(lse, ref, what):
    assert np.all(np.isfinite(lse)), f"{what}: non-finite lse"
    max_abs, _ = metrics(lse, ref)
    log(f"  {what}: lse max_abs={max_abs:.3e}")
    assert max_abs <= LSE_MAX_ABS, (what, max_abs)


def row_errors(g, ref, allow=None):
    """Per-row L2 error of g against ref, less the row's allowance (if any),
    relative to max(row norm, rms row norm)."""
    g = np.asarray(g, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(g.shape)
    if ref.size == 0:
        return np.zeros(0)
    rown = np.linalg.norm(ref, axis=1)
    rms = float(np.linalg.norm(ref)) / np.sqrt(ref.shape[0])
    floor = np.maximum(rown, rms)
    err = np.linalg.norm(g - ref, axis=1)
    if allow is not None:
        err = np.maximum(err - np.asarray(allow, dtype=np.float64).reshape(-1), 0.0)
    return np.where(floor > 0, err / np.where(floor > 0, floor, 1.0), err)


def dq_allowance(q, k, v, do, scale, causal, block_mask=None):
    """Per-row bound (L2) on how far dQ_i moves because D_i = sum_k dO_ik O_ik
    is formed from the forward's stored O rather than the exact one, for one
    head, from the oracle alone. dQ_i is linear in D_i with slope
    -scale * sum_j P_ij K_j = -scale * (attention of q over values K)_i, and
    the stored O differs from the exact one by its bf16 rounding (u |O_ik|)
    plus that of the probabilities it was formed from (u sum_j P_ij |V_jk|),
    u = 2^-8, so |delta D_i| <= u sum_k |dO_ik| (|O_ik| + sum_j P_ij |V_jk|)."""
    o, _ = oracle.forward_head(q, k, v, scale, causal, block_mask=block_mask)
    pav, _ = oracle.forward_head(q, k, np.abs(v), scale, causal, block_mask=block_mask)
    pk, _ = oracle.forward_head(q, k, k, scale, causal, block_mask=block_mask)
    dmax = BF16_U * np.sum(np.abs(do) * (np.abs(o) + pav), axis=1)
    return abs(scale) * dmax * np.linalg.norm(pk, axis=1)


def dq_allowances(q, k, v, do, scale, causal, block_mask=None):
    """dq_allowance for every query head of [B,H,N,d] q, do and [B,Hkv,N,d]
    k, v (query head h reads K/V head h / (H / Hkv)); block_mask as for
    oracle.backward. Returns [B, H, N]."""
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    out = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(H):
            g = oracle.kv_head(h, H, Hkv)
            bm = None if block_mask is None else (
                np.asarray(block_mask) if np.ndim(block_mask) == 2 else np.asarray(block_mask)[b, h])
            out[b, h] = dq_allowance(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal, bm)
    return out


def check_grad(g, ref, what, allow=None):
    """Head-level relative L2 and the per-row bound; `allow`: an additive
    per-row allowance (dq_allowance for dQ)."""
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    max_abs, rel = metrics(g, ref)
    rows = row_errors(g, ref, allow)
    worst = float(rows.max()) if rows.size else 0.0
    log(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} worst row={worst:.3e}")
    assert rel <= GRAD_REL_L2, (what, max_abs, rel)
    assert worst <= GRAD_ROW_REL, (what, "row", int(np.argmax(rows)), worst)


def sample_rows(n, seed, edge=256, rand=512):
    """First and last `edge` rows plus `rand` seeded random rows, sorted, unique."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(edge, n))) | set(range(max(0, n - edge), n))
    rows |= set(rng.integers(0, n, size=min(rand, n)).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def sample_heads(B, H, count, seed):
    rng = np.random.default_rng(seed)
    total = B * H
    picks = [0, total - 1] + rng.integers(0, total, size=max(0, count - 2)).tolist()
    seen = []
    for p in picks:
        if p not in seen:
            seen.append(p)
    return [(p // H, p % H) for p in seen[:count]]
