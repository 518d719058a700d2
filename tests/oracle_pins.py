"""Checks that pin the fp64 oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix. They look the oracle functions up on
the module at call time, so tests/test_oracle_mutations.py can plant a
mistake in the oracle and confirm that at least one pin catches it.

Sources of truth used here, none of which is the oracle's own code:
* hand-derived closed forms (tests/golden/closed_form.json);
* torch's fp64 CPU scaled_dot_product_attention and autograd (a library);
* central finite differences of the oracle's forward (for its backward);
* pure-Python loops with math.exp on tiny inputs (brute force);
* the blockwise online-softmax algorithm of the unite.ai page ("Dettagli di
  Implementazione"), written here independently, with the old running sum
  restored in the output update (the printed version omits it);
* invariants of softmax attention (rows of P sum to 1, a single key returns
  V, constant V returns that constant, zero queries give (prefix) means,
  the merge identity over a split key set, shift and permutation behaviour,
  and the gradient identities sum_j dK_j = 0, sum_j dV_j = sum_i dO_i).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle.attention as A
import oracle.fp8 as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_form.json")


def _close(x, y, tol, what):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, f"{what}: shape {x.shape} vs {y.shape}"
    err = np.max(np.abs(x - y)) if x.size else 0.0
    assert np.all(np.isfinite(x)) and err <= tol, f"{what}: max abs err {err} > {tol}"


def _rand_head(rng, n, d, nk=None):
    nk = n if nk is None else nk
    return (rng.standard_normal((n, d)), rng.standard_normal((nk, d)),
            rng.standard_normal((nk, d)))


# ---------------------------------------------------------------- golden

def pin_golden_forward():
    data = json.load(open(GOLDEN))
    for case in data["cases"]:
        o, lse = A.forward_head(np.array(case["q"]), np.array(case["k"]),
                                np.array(case["v"]), case["scale"], case["causal"])
        _close(o, case["o"], 1e-12, case["name"] + " O")
        _close(lse, case["lse"], 1e-12, case["name"] + " lse")


def pin_golden_backward():
    data = json.load(open(GOLDEN))
    for case in data["backward_cases"]:
        q, k, v, do = (np.array(case[x]) for x in ("q", "k", "v", "do"))
        o, _ = A.forward_head(q, k, v, case["scale"], case["causal"])
        _close(o, case["o"], 1e-12, case["name"] + " O")
        dq, dk, dv = A.backward_head(q, k, v, do, case["scale"], case["causal"])
        _close(dq, case["dq"], 1e-12, case["name"] + " dQ")
        _close(dk, case["dk"], 1e-12, case["name"] + " dK")
        _close(dv, case["dv"], 1e-12, case["name"] + " dV")


# ---------------------------------------------------------------- library

SHAPES = [(1, 1), (2, 3), (5, 4), (17, 8), (33, 16), (64, 5)]


def _torch_sdpa(q, k, v, scale, causal):
    t = [torch.tensor(x, dtype=torch.float64)[None, None] for x in (q, k, v)]
    if scale >= 0:
        return torch.nn.functional.scaled_dot_product_attention(
            *t, is_causal=causal, scale=scale)[0, 0].numpy()
    # torch's fused path masks before scaling, which turns -inf into +inf for a
    # negative scale; form the masked scores and call torch.softmax instead.
    s = (t[0] @ t[1].transpose(-1, -2))[0, 0] * scale
    if causal:
        n = s.shape[0]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -math.inf)
    return (torch.softmax(s, dim=-1) @ t[2][0, 0]).numpy()


def pin_vs_torch_sdpa():
    rng = np.random.default_rng(11)
    for n, d in SHAPES:
        for causal in (False, True):
            for scale in (1.0 / math.sqrt(d), -0.7, 2.5):
                q, k, v = _rand_head(rng, n, d)
                o, lse = A.forward_head(q, k, v, scale, causal)
                _close(o, _torch_sdpa(q, k, v, scale, causal), 1e-12,
                       f"O vs torch n={n} d={d} causal={causal} scale={scale}")
                s = torch.tensor(q) @ torch.tensor(k).T * scale
                if causal:
                    s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -math.inf)
                _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12,
                       f"lse vs torch.logsumexp n={n} d={d}")


def pin_backward_vs_autograd():
    rng = np.random.default_rng(12)
    for n, d in SHAPES:
        for causal in (False, True):
            scale = 1.0 / math.sqrt(d)
            q, k, v = _rand_head(rng, n, d)
            do = rng.standard_normal((n, d))
            t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
            out = torch.nn.functional.scaled_dot_product_attention(
                t[0][None, None], t[1][None, None], t[2][None, None],
                is_causal=causal, scale=scale)[0, 0]
            out.backward(torch.tensor(do))
            dq, dk, dv = A.backward_head(q, k, v, do, scale, causal)
            for name, mine, ref in (("dQ", dq, t[0].grad), ("dK", dk, t[1].grad),
                                    ("dV", dv, t[2].grad)):
                _close(mine, ref.numpy(), 1e-11, f"{name} vs autograd n={n} causal={causal}")


# ---------------------------------------------------------------- finite differences

def pin_finite_differences():
    rng = np.random.default_rng(13)
    eps = 1e-6
    for n, d, causal in ((3, 2, False), (4, 3, True), (1, 2, True)):
        scale = 0.8
        q, k, v = _rand_head(rng, n, d)
        do = rng.standard_normal((n, d))
        grads = A.backward_head(q, k, v, do, scale, causal)

        def loss(qq, kk, vv):
            return float(np.sum(do * A.forward_head(qq, kk, vv, scale, causal)[0]))

        for which in range(3):
            base = [q, k, v]
            num = np.zeros_like(base[which])
            for idx in np.ndindex(*num.shape):
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][idx] += eps
                minus[which][idx] -= eps
                num[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
            _close(grads[which], num, 1e-7, f"finite differences input {which} n={n}")


# ---------------------------------------------------------------- brute force

def pin_brute_force():
    rng = np.random.default_rng(14)
    for n, d in ((1, 1), (3, 2), (6, 3)):
        for causal in (False, True):
            scale = 0.9
            q, k, v = _rand_head(rng, n, d)
            o, lse = A.forward_head(q, k, v, scale, causal)
            for i in range(n):
                keys = [j for j in range(n) if (j <= i or not causal)]
                scores = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
                weights = [math.exp(s) for s in scores]
                total = sum(weights)
                for c in range(d):
                    ref = sum(w * v[j][c] for w, j in zip(weights, keys)) / total
                    assert abs(o[i][c] - ref) <= 1e-12, ("brute O", n, i, c)
                assert abs(lse[i] - math.log(total)) <= 1e-12, ("brute lse", n, i)


# ---------------------------------------------------------------- online recurrence

def online_blockwise(q, k, v, scale, causal, block):
    """Blockwise attention with a running max and sum, Q blocks outer, K/V inner.

    Follows the steps of the unite.ai page's simplified implementation, with
    the output update written as O <- (e^(m-m_new) * l_old * O + P V) / l_new,
    i.e. with the old running sum restored, which the printed code omits.
    """
    n = q.shape[0]
    out = np.zeros((n, v.shape[1]))
    run_l = np.zeros(n)
    run_m = np.full(n, -np.inf)
    for i0 in range(0, n, block):
        rows = np.arange(i0, min(n, i0 + block))
        for j0 in range(0, k.shape[0], block):
            cols = np.arange(j0, min(k.shape[0], j0 + block))
            s = scale * (q[rows] @ k[cols].T)
            if causal:
                s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
            m_new = np.maximum(run_m[rows], s.max(axis=1))
            live = np.isfinite(m_new)
            m_use = np.where(live, m_new, 0.0)
            p = np.exp(s - m_use[:, None])
            alpha = np.where(np.isfinite(run_m[rows]), np.exp(run_m[rows] - m_use), 0.0)
            l_new = alpha * run_l[rows] + p.sum(axis=1)
            safe = np.where(l_new > 0, l_new, 1.0)
            out[rows] = ((alpha * run_l[rows])[:, None] * out[rows] + p @ v[cols]) / safe[:, None]
            run_l[rows] = l_new
            run_m[rows] = np.where(live, m_new, run_m[rows])
    return out, run_m + np.log(run_l)


def pin_online_recurrence():
    rng = np.random.default_rng(15)
    for n, d, block in ((64, 8, 16), (50, 4, 7), (130, 16, 32)):
        for causal in (False, True):
            q, k, v = _rand_head(rng, n, d)
            q *= 3.0  # peaked rows: the running max moves between blocks
            o, lse = A.forward_head(q, k, v, 0.5, causal)
            o2, lse2 = online_blockwise(q, k, v, 0.5, causal, block)
            _close(o, o2, 1e-12, f"online recurrence O n={n} block={block}")
            _close(lse, lse2, 1e-12, f"online recurrence lse n={n}")


# ---------------------------------------------------------------- invariants

def pin_forward_invariants():
    rng = np.random.default_rng(16)
    n, d = 40, 6
    for causal in (False, True):
        q, k, v = _rand_head(rng, n, d)
        scale = 0.6
        # rows of P sum to one
        p = A.probabilities_head(q, k, scale, causal)
        _close(p.sum(axis=1), np.ones(n), 1e-12, "P row sums")
        if causal:
            assert np.all(np.triu(p, 1) == 0.0), "causal P has mass above the diagonal"
        # constant V returns the constant
        cv = np.tile(rng.standard_normal(d), (n, 1))
        _close(A.forward_head(q, k, cv, scale, causal)[0], cv, 1e-12, "constant V")
        # zero queries: (prefix) means, lse = ln(count)
        o0, l0 = A.forward_head(np.zeros_like(q), k, v, scale, causal)
        if causal:
            means = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
            counts = np.arange(1, n + 1)
        else:
            means = np.tile(v.mean(axis=0), (n, 1))
            counts = np.full(n, n)
        _close(o0, means, 1e-12, "zero query means")
        _close(l0, np.log(counts), 1e-12, "zero query lse")
        # key shift: O unchanged, lse shifts by scale * q.c
        c = rng.standard_normal(d)
        o, lse = A.forward_head(q, k, v, scale, causal)
        o_s, lse_s = A.forward_head(q, k + c, v, scale, causal)
        _close(o_s, o, 1e-11, "key shift O")
        _close(lse_s, lse + scale * (q @ c), 1e-11, "key shift lse")
    # single key returns V exactly
    q, k, v = _rand_head(rng, 5, d, nk=1)
    o, lse = A.forward_head(q, k, v, 1.3, False)
    _close(o, np.tile(v, (5, 1)), 0.0, "single key")
    _close(lse, 1.3 * (q @ k[0]), 1e-12, "single key lse")
    # joint permutation of K and V rows (non-causal) leaves O unchanged
    q, k, v = _rand_head(rng, 30, d)
    perm = rng.permutation(30)
    _close(A.forward_head(q, k[perm], v[perm], 0.4, False)[0],
           A.forward_head(q, k, v, 0.4, False)[0], 1e-12, "permutation")
    # split the key set in two and merge the partial results
    q, k, v = _rand_head(rng, 24, d, nk=50)
    q *= 4.0
    o, lse = A.forward_head(q, k, v, 0.7, False)
    o1, l1 = A.forward_head(q, k[:13], v[:13], 0.7, False)
    o2, l2 = A.forward_head(q, k[13:], v[13:], 0.7, False)
    om, lm = A.merge(o1, l1, o2, l2)
    _close(om, o, 1e-12, "merge O")
    _close(lm, lse, 1e-12, "merge lse")


def pin_backward_invariants():
    rng = np.random.default_rng(17)
    n, d = 30, 5
    for causal in (False, True):
        q, k, v = _rand_head(rng, n, d)
        do = rng.standard_normal((n, d))
        dq, dk, dv = A.backward_head(q, k, v, do, 0.5, causal)
        # softmax is invariant to shifting all keys: the key gradients sum to zero
        _close(dk.sum(axis=0), np.zeros(d), 1e-11, "sum dK")
        # each row of P sums to one: the value gradients sum to the sum of dO
        _close(dv.sum(axis=0), do.sum(axis=0), 1e-11, "sum dV")
        # identical keys: scores do not depend on q, so dQ = 0
        kk = np.tile(k[:1], (n, 1))
        dq0, _, _ = A.backward_head(q, kk, v, do, 0.5, causal)
        _close(dq0, np.zeros_like(dq0), 1e-12, "identical keys dQ")
        # D_i = sum_k dO_ik O_ik equals sum_j P_ij dP_ij
        p = A.probabilities_head(q, k, 0.5, causal)
        o = A.forward_head(q, k, v, 0.5, causal)[0]
        _close((do * o).sum(axis=1), (p * (do @ v.T)).sum(axis=1), 1e-11, "D identity")


# ---------------------------------------------------------------- grouped K/V heads

GQA_SHAPES = ((1, 4, 2, 5, 3), (2, 6, 3, 4, 2), (1, 3, 1, 6, 4), (1, 2, 2, 3, 2))


def _torch_gqa(q, k, v, do, scale, causal):
    """torch fp64 autograd with each K/V head copied to its query heads by
    repeat_interleave (consecutive groups); autograd sums the copies'
    gradients."""
    heads, kv_heads = q.shape[1], k.shape[1]
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    ke = tk.repeat_interleave(heads // kv_heads, dim=1)
    ve = tv.repeat_interleave(heads // kv_heads, dim=1)
    s = torch.matmul(tq, ke.transpose(-1, -2)) * scale
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -math.inf)
    o = torch.matmul(torch.softmax(s, dim=-1), ve)
    (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_gqa_vs_autograd():
    rng = np.random.default_rng(21)
    for bsz, heads, kv_heads, n, d in GQA_SHAPES:
        for causal in (False, True):
            q = rng.standard_normal((bsz, heads, n, d))
            k = rng.standard_normal((bsz, kv_heads, n, d))
            v = rng.standard_normal((bsz, kv_heads, n, d))
            do = rng.standard_normal((bsz, heads, n, d))
            o, _ = A.forward(q, k, v, 0.6, causal)
            grads = A.backward(q, k, v, do, 0.6, causal)
            ref = _torch_gqa(q, k, v, do, 0.6, causal)
            what = f"H={heads} Hkv={kv_heads} causal={causal}"
            _close(o, ref[0], 1e-12, f"grouped O vs torch {what}")
            for name, mine, r in zip(("dQ", "dK", "dV"), grads, ref[1:]):
                _close(mine, r, 1e-11, f"grouped {name} vs autograd {what}")


def pin_gqa_finite_differences():
    rng = np.random.default_rng(22)
    eps = 1e-6
    for heads, kv_heads, causal in ((4, 2, True), (3, 1, False)):
        n, d, scale = 3, 2, 0.9
        q = rng.standard_normal((1, heads, n, d))
        k = rng.standard_normal((1, kv_heads, n, d))
        v = rng.standard_normal((1, kv_heads, n, d))
        do = rng.standard_normal((1, heads, n, d))
        grads = A.backward(q, k, v, do, scale, causal)

        def loss(qq, kk, vv):
            return float(np.sum(do * A.forward(qq, kk, vv, scale, causal)[0]))

        for which in (1, 2):  # the shared K and V
            base = [q, k, v]
            num = np.zeros_like(base[which])
            for idx in np.ndindex(*num.shape):
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][idx] += eps
                minus[which][idx] -= eps
                num[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
            _close(grads[which], num, 1e-7,
                   f"grouped finite differences input {which} H={heads} Hkv={kv_heads}")


# ---------------------------------------------------------------- local (sliding-window) masks

WINDOWS = ((0, 0), (3, 0), (2, 1), (-1, 2), (4, -1), (1, 5), (0, -1))


def _torch_window_mask(n, left, right):
    """Visible-key mask built from torch.tril / torch.triu (no index arithmetic)."""
    ones = torch.ones(n, n, dtype=torch.bool)
    mask = ones.clone()
    if right >= 0:
        mask &= ones.tril(right)
    if left >= 0:
        mask &= ones.triu(-left)
    return mask


def pin_window_special_cases():
    rng = np.random.default_rng(31)
    for n, d in ((7, 3), (12, 5)):
        q, k, v = _rand_head(rng, n, d)
        for scale in (0.6, -1.3):
            # (-1, 0) is the causal mask, (-1, -1) none at all: exactly the same arithmetic
            for win, flag in (((-1, 0), True), ((-1, -1), False)):
                o1, l1 = A.forward_head(q, k, v, scale, win)
                o2, l2 = A.forward_head(q, k, v, scale, flag)
                assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"window {win}"
            # (0, 0): every row sees only its own key
            o, lse = A.forward_head(q, k, v, scale, (0, 0))
            _close(o, v, 1e-14, "window (0,0) returns V")
            _close(lse, scale * np.sum(q * k, axis=1), 1e-13, "window (0,0) lse")


def pin_window_vs_torch():
    rng = np.random.default_rng(32)
    for n, d in ((9, 4), (16, 3)):
        for left, right in WINDOWS:
            q, k, v = _rand_head(rng, n, d)
            do = rng.standard_normal((n, d))
            scale = 0.7
            mask = _torch_window_mask(n, left, right)
            t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
            sc = (t[0] @ t[1].T * scale).masked_fill(~mask, -math.inf)
            o_t = torch.softmax(sc, dim=-1) @ t[2]
            (o_t * torch.tensor(do)).sum().backward()
            o, lse = A.forward_head(q, k, v, scale, (left, right))
            what = f"window ({left},{right}) n={n}"
            _close(o, o_t.detach().numpy(), 1e-12, f"O vs torch {what}")
            _close(lse, torch.logsumexp(sc, dim=-1).detach().numpy(), 1e-12, f"lse vs torch {what}")
            grads = A.backward_head(q, k, v, do, scale, (left, right))
            for name, mine, ref in zip(("dQ", "dK", "dV"), grads, t):
                _close(mine, ref.grad.numpy(), 1e-11, f"{name} vs autograd {what}")


def pin_window_brute_force():
    rng = np.random.default_rng(33)
    n, d, scale = 6, 2, 0.9
    for left, right in WINDOWS:
        q, k, v = _rand_head(rng, n, d)
        o, lse = A.forward_head(q, k, v, scale, (left, right))
        for i in range(n):
            keys = [j for j in range(n)
                    if (left < 0 or i - left <= j) and (right < 0 or j <= i + right)]
            w = [math.exp(scale * sum(q[i, c] * k[j, c] for c in range(d))) for j in keys]
            tot = sum(w)
            for c in range(d):
                ref = sum(wj * v[j, c] for wj, j in zip(w, keys)) / tot
                assert abs(o[i, c] - ref) < 1e-12, f"brute force window ({left},{right}) row {i}"
            assert abs(lse[i] - math.log(tot)) < 1e-12


# ---------------------------------------------------------------- block-sparse masks
# A mask over blocks of 128 query rows x 128 keys (the reading stated in
# oracle/attention.py); the pins expand it element by element themselves.

BLOCK = 128


def _expand_block_mask(bm, n):
    keep = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            keep[i, j] = bm[i // BLOCK][j // BLOCK] != 0
    return keep


def _window_keep(n, left, right):
    keep = np.ones((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            keep[i, j] = (left < 0 or j >= i - left) and (right < 0 or j <= i + right)
    return keep


def _random_block_mask(rng, nb, diagonal=True):
    bm = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
    if diagonal:
        np.fill_diagonal(bm, 1)
    return bm


def pin_block_mask_all_ones():
    # an all-ones block mask is no block mask at all: the same arithmetic, bitwise
    rng = np.random.default_rng(41)
    n, d = 300, 6
    q, k, v = _rand_head(rng, n, d)
    do = rng.standard_normal((n, d))
    for causal in (True, False, (40, 7)):
        ones = np.ones((3, 3), dtype=np.uint8)
        o1, l1 = A.forward_head(q, k, v, 0.4, causal)
        o2, l2 = A.forward_head(q, k, v, 0.4, causal, block_mask=ones)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), f"all-ones mask {causal}"
        for g1, g2 in zip(A.backward_head(q, k, v, do, 0.4, causal),
                          A.backward_head(q, k, v, do, 0.4, causal, block_mask=ones)):
            assert np.array_equal(g1, g2), f"all-ones mask gradients {causal}"


def pin_block_mask_vs_torch():
    rng = np.random.default_rng(42)
    n, d, scale = 300, 8, 0.5
    for causal, (left, right) in ((True, (-1, 0)), (False, (-1, -1)), ((60, 20), (60, 20))):
        q, k, v = _rand_head(rng, n, d)
        do = rng.standard_normal((n, d))
        bm = _random_block_mask(rng, 3)  # the diagonal blocks keep every row non-empty
        keep = torch.tensor(_expand_block_mask(bm, n) & _window_keep(n, left, right))
        t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
        sc = (t[0] @ t[1].T * scale).masked_fill(~keep, -math.inf)
        o_t = torch.softmax(sc, dim=-1) @ t[2]
        (o_t * torch.tensor(do)).sum().backward()
        o, lse = A.forward_head(q, k, v, scale, causal, block_mask=bm)
        what = f"block mask {bm.tolist()} {causal}"
        _close(o, o_t.detach().numpy(), 1e-12, f"O vs torch {what}")
        _close(lse, torch.logsumexp(sc, dim=-1).detach().numpy(), 1e-12, f"lse vs torch {what}")
        grads = A.backward_head(q, k, v, do, scale, causal, block_mask=bm)
        for name, mine, ref in zip(("dQ", "dK", "dV"), grads, t):
            _close(mine, ref.grad.numpy(), 1e-11, f"{name} vs autograd {what}")
        # per-head masks through the batched calls
        qb, kb, vb, dob = (np.stack([x, x[::-1].copy()])[None] for x in (q, k, v, do))
        masks = np.stack([bm, bm.T])[None]
        ob, lb = A.forward(qb, kb, vb, scale, causal, block_mask=masks)
        _close(ob[0, 0], o, 1e-15, f"batched head 0 {what}")
        o1, _ = A.forward_head(qb[0, 1], kb[0, 1], vb[0, 1], scale, causal, block_mask=bm.T)
        _close(ob[0, 1], o1, 1e-15, f"batched head 1 {what}")


def pin_block_mask_brute_force():
    rng = np.random.default_rng(43)
    n, d, scale = 260, 2, 0.8  # three blocks, the last one 4 rows
    q, k, v = _rand_head(rng, n, d)
    bm = _random_block_mask(rng, 3)
    for causal in (True, False):
        o, lse = A.forward_head(q, k, v, scale, causal, block_mask=bm)
        for i in (0, 5, 127, 128, 200, 255, 256, 259):
            keys = [j for j in range(n) if bm[i // BLOCK][j // BLOCK] and (not causal or j <= i)]
            w = [math.exp(scale * sum(q[i, c] * k[j, c] for c in range(d))) for j in keys]
            tot = sum(w)
            for c in range(d):
                ref = sum(wj * v[j, c] for wj, j in zip(w, keys)) / tot
                assert abs(o[i, c] - ref) < 1e-12, f"brute force block mask row {i} {causal}"
            assert abs(lse[i] - math.log(tot)) < 1e-12


def pin_block_mask_empty_rows():
    # query block 1 sees nothing: its O is 0, its lse -inf, its dQ 0; the
    # other rows and every dK, dV are those of attention over the other rows
    # alone (torch, which cannot take an empty row)
    rng = np.random.default_rng(44)
    n, d, scale = 300, 5, 0.6
    q, k, v = _rand_head(rng, n, d)
    do = rng.standard_normal((n, d))
    bm = np.array([[1, 0, 1], [0, 0, 0], [0, 1, 1]], dtype=np.uint8)
    o, lse = A.forward_head(q, k, v, scale, False, block_mask=bm)
    empty = np.arange(128, 256)
    live = np.concatenate([np.arange(128), np.arange(256, n)])
    assert np.all(o[empty] == 0.0) and np.all(lse[empty] == -np.inf), "empty rows"
    dq, dk, dv = A.backward_head(q, k, v, do, scale, False, block_mask=bm)
    assert np.all(dq[empty] == 0.0), "no gradient through an empty row"
    keep = torch.tensor(_expand_block_mask(bm, n)[live])
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q[live], k, v)]
    sc = (t[0] @ t[1].T * scale).masked_fill(~keep, -math.inf)
    o_t = torch.softmax(sc, dim=-1) @ t[2]
    (o_t * torch.tensor(do[live])).sum().backward()
    _close(o[live], o_t.detach().numpy(), 1e-12, "live rows O")
    _close(dq[live], t[0].grad.numpy(), 1e-11, "live rows dQ")
    _close(dk, t[1].grad.numpy(), 1e-11, "dK from the live rows")
    _close(dv, t[2].grad.numpy(), 1e-11, "dV from the live rows")


def pin_block_diagonal_segments():
    # a block-diagonal mask is independent attention over each 128-row segment
    rng = np.random.default_rng(45)
    n, d, scale = 384, 4, 0.7
    q, k, v = _rand_head(rng, n, d)
    do = rng.standard_normal((n, d))
    eye = np.eye(3, dtype=np.uint8)
    o, lse = A.forward_head(q, k, v, scale, False, block_mask=eye)
    grads = A.backward_head(q, k, v, do, scale, False, block_mask=eye)
    for s in range(3):
        seg = slice(s * BLOCK, (s + 1) * BLOCK)
        os_, ls_ = A.forward_head(q[seg], k[seg], v[seg], scale, False)
        _close(o[seg], os_, 1e-14, f"segment {s} O")
        _close(lse[seg], ls_, 1e-14, f"segment {s} lse")
        for g, gs in zip(grads, A.backward_head(q[seg], k[seg], v[seg], do[seg], scale, False)):
            _close(g[seg], gs, 1e-13, f"segment {s} gradients")


# ---------------------------------------------------------------- row chunks and row subsets
# forward_head forms the scores of at most 512 query rows at a time and can
# compute a subset of the rows. Every GPU comparison at N > 512 goes through
# these two paths, so they are pinned at a length that takes three chunks
# (512 + 512 + 76 rows), with every kind of mask, against torch fp64
# attention whose masks are built from tril / triu / kron alone.

def _torch_masked_attention(q, k, v, scale, keep):
    t = [torch.tensor(x, dtype=torch.float64) for x in (q, k, v)]
    sc = (t[0] @ t[1].T * scale).masked_fill(~keep, -math.inf)
    return (torch.softmax(sc, dim=-1) @ t[2]).numpy(), torch.logsumexp(sc, dim=-1).numpy()


def _kron_block_keep(bm, n):
    """Element mask of a block mask by a Kronecker product with 128 x 128 ones."""
    return torch.tensor(np.kron(np.asarray(bm) != 0, np.ones((BLOCK, BLOCK), dtype=bool))[:n, :n])


def pin_row_chunks_vs_torch():
    rng = np.random.default_rng(47)
    n, d, scale = 1100, 4, 0.8
    nb = -(-n // BLOCK)
    subset = np.concatenate([[1099, 0, 512, 511, 1024, 1023, 700], rng.permutation(n)[:650],
                             [5, 5]])  # unsorted, across every chunk edge, one row twice
    cases = [(True, _torch_window_mask(n, -1, 0), None),
             ((300, 50), _torch_window_mask(n, 300, 50), None),
             ((-1, 7), _torch_window_mask(n, -1, 7), None),
             ((600, -1), _torch_window_mask(n, 600, -1), None)]
    bm = _random_block_mask(rng, nb)  # diagonal blocks kept: no row is empty
    cases.append((True, _torch_window_mask(n, -1, 0) & _kron_block_keep(bm, n), bm))
    cases.append((False, _kron_block_keep(bm.T, n), bm.T.copy()))
    for causal, keep, mask in cases:
        q, k, v = _rand_head(rng, n, d)
        ro, rl = _torch_masked_attention(q, k, v, scale, keep)
        what = f"n={n} mask={causal} block={mask is not None}"
        o, lse = A.forward_head(q, k, v, scale, causal, block_mask=mask)
        _close(o, ro, 1e-12, f"chunked O vs torch {what}")
        _close(lse, rl, 1e-12, f"chunked lse vs torch {what}")
        o_s, lse_s = A.forward_head(q, k, v, scale, causal, rows=subset, block_mask=mask)
        _close(o_s, ro[subset], 1e-12, f"row subset O vs torch {what}")
        _close(lse_s, rl[subset], 1e-12, f"row subset lse vs torch {what}")


def pin_row_chunks_zero_queries():
    # closed form across chunks: zero queries see the mean of their visible
    # values, lse = ln(count), for a causal mask and a window
    rng = np.random.default_rng(48)
    n, d = 1100, 3
    v = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    q = np.zeros((n, d))
    rows = np.array([1099, 3, 600, 1030, 512])
    for left, right in ((-1, 0), (100, 20)):
        o, lse = A.forward_head(q, k, v, 1.0, (left, right), rows=rows)
        for r, i in enumerate(rows):
            lo = 0 if left < 0 else max(0, i - left)
            hi = min(n - 1, i + right)
            _close(o[r], v[lo:hi + 1].mean(axis=0), 1e-12, f"zero-query mean row {i}")
            _close(lse[r], math.log(hi - lo + 1), 1e-12, f"zero-query lse row {i}")


# ---------------------------------------------------------------- FP8 with incoherent processing

def pin_fp8_e4m3_golden():
    data = json.load(open(os.path.join(os.path.dirname(GOLDEN), "fp8_e4m3.json")))
    for case in data["cases"]:
        got = float(F.e4m3_round(case["x"]))
        assert got == case["q"], f"e4m3({case['x']}) = {got}, expected {case['q']} ({case['why']})"


def pin_fp8_e4m3_grid():
    vals = F.e4m3_values()
    assert len(vals) == 127 and vals[-1] == 448.0 and np.all(np.diff(vals) > 0)
    # every representable value is a fixed point, with either sign
    assert np.array_equal(F.e4m3_round(vals), vals)
    assert np.array_equal(F.e4m3_round(-vals), -vals)
    # a midpoint goes to the neighbour with the even mantissa (grid index even)
    mids = (vals[:-1] + vals[1:]) / 2
    want = np.where(np.arange(len(mids)) % 2 == 0, vals[:-1], vals[1:])
    assert np.array_equal(F.e4m3_round(mids), want)
    # just inside a midpoint goes to the nearer value
    eps = np.diff(vals) * 1e-3
    assert np.array_equal(F.e4m3_round(mids - eps), vals[:-1])
    assert np.array_equal(F.e4m3_round(mids + eps), vals[1:])


def pin_fp8_scales():
    """Power-of-two scales, worked by hand: the smallest 2^e with max / 2^e <= 448."""
    got = F.pow2_scale(np.array([448.0, 449.0, 224.0, 224.5, 0.0, 1e-3]))
    assert np.array_equal(got, [1.0, 2.0, 0.5, 1.0, 1.0, 2.0 ** -18]), got
    x = np.zeros((130, 8))
    x[5, 3] = 1000.0          # tile 0: 1000 / 448 = 2.23 -> 4
    x[74, 0] = -0.5           # tile 1: 0.5 / 448 = 2^-9.81 -> 2^-9
    x[128:, 1] = 3.0          # tile 2 (ragged, 2 rows): 3 / 448 = 2^-7.22 -> 2^-7
    codes, b = F.quantize_tiles(x)
    assert np.array_equal(b, np.repeat([4.0, 2.0 ** -9, 2.0 ** -7], [64, 64, 2]))
    assert codes[5, 3] == 256.0 and codes[74, 0] == -256.0 and codes[129, 1] == 384.0
    codes, a = F.quantize_rows(x)
    assert a[5] == 4.0 and a[74] == 2.0 ** -9 and a[0] == 1.0 and a[129] == 2.0 ** -7
    assert codes[5, 3] == 256.0


def pin_fp8_forward_golden():
    data = json.load(open(os.path.join(os.path.dirname(GOLDEN), "fp8_forward.json")))
    for case in data["cases"]:
        o, lse = F.forward_fp8_head(np.array(case["q"]), np.array(case["k"]), np.array(case["v"]),
                                    case["scale"], False)
        _close(o, case["o"], 1e-12, case["name"] + " O")
        _close(lse, case["lse"], 1e-12, case["name"] + " lse")


def pin_fp8_v_blocks():
    """V scales per column and block of 32 consecutive keys, worked by hand."""
    x = np.zeros((70, 3))
    x[3, 0] = 1000.0     # column 0, keys 0-31: 1000 / 448 -> 4
    x[40, 0] = 0.5       # column 0, keys 32-63: 0.5 / 448 = 2^-9.81 -> 2^-9
    x[69, 2] = -3.0      # column 2, keys 64-69 (ragged): 3 / 448 -> 2^-7
    codes, sc = F.quantize_key_blocks(x)
    assert np.array_equal(sc[:32, 0], np.full(32, 4.0)) and np.array_equal(sc[32:64, 0], np.full(32, 2.0 ** -9))
    assert np.array_equal(sc[64:, 0], np.ones(6)) and np.array_equal(sc[:, 1], np.ones(70))
    assert np.array_equal(sc[64:, 2], np.full(6, 2.0 ** -7)) and sc[0, 2] == 1.0
    assert codes[3, 0] == 256.0 and codes[40, 0] == 256.0 and codes[69, 2] == -384.0


def pin_fp8_pv_error_bound():
    """Given the FP8 scores S, the FP8 second product errs by at most
    sum_j |P~_ij V~_jc - P_ij V_jc| / l_i, bounded term by term with the
    e4m3 rounding errors: relative 2^-4 (normals), absolute 2^-18 (P, rounded
    with the scale 2^-8, below 2^-14) and 2^-10 times the block scale (V)."""
    rng = np.random.default_rng(44)
    n, d, scale = 90, 64, 0.125
    q, k, v = _rand_head(rng, n, d)
    v[:, 5] *= 40.0
    for causal in (False, True):
        s = F.fp8_scores(q, k, scale)
        if causal:
            s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
        # the probabilities relative to the row maximum rounded up to a power of two
        m = np.ceil(np.max(s, axis=1, keepdims=True) / np.log(2.0))
        p = np.exp2(s / np.log(2.0) - m)
        l = np.sum(p, axis=1, keepdims=True)
        exact = (p @ v) / l
        _, bs = F.quantize_key_blocks(v)
        av = np.abs(v)
        per = (p @ av) * (2.0 ** -3 + 2.0 ** -8) + 2.0 ** -18 * 1.07 * (np.ones_like(p) @ av) \
            + 1.07 * 2.0 ** -10 * (p @ bs) + 2.0 ** -28 * (np.ones_like(p) @ bs)
        got, _ = F.forward_fp8_head(q, k, v, scale, causal)
        err = np.abs(got - exact)
        assert np.all(err <= per / l), "fp8 P V error bound"
        assert np.max(err) > 0.0


def pin_fp8_hadamard():
    for d in (1, 2, 64, 128):
        h = F.hadamard(d)
        assert np.all(np.abs(h) == 1.0)
        assert np.array_equal(h @ h.T, d * np.eye(d))


def pin_fp8_rotation_is_exact():
    """Without quantisation the random-sign Hadamard changes no score:
    (Q diag(s) H)(K diag(s) H)^T / d = Q K^T."""
    rng = np.random.default_rng(41)
    for n, d in ((40, 64), (70, 128)):
        q, k, v = _rand_head(rng, n, d)
        signs = rng.choice([-1.0, 1.0], size=d)
        s_rot = F.fp8_scores(q, k, 0.3, signs, quantize=False)
        _close(s_rot, 0.3 * (q @ k.T), 1e-12, f"rotated scores d={d}")
        o, lse = F.forward_fp8_head(q, k, v, 0.3, True, signs, quantize=False)
        ro, rl = A.forward_head(q, k, v, 0.3, True)
        _close(o, ro, 1e-12, f"rotated forward O d={d}")
        _close(lse, rl, 1e-12, f"rotated forward lse d={d}")


def pin_fp8_error_bound():
    """Each quantised operand is within 2^-4 (relative, normals) plus 2^-10
    (absolute, subnormals, in units of its scale) of the exact value, so a
    score errs by at most sum_c |q~_c| |k~_c| (2^-3 + 2^-8) plus the subnormal
    terms, times scale / d for the rotated form."""
    rng = np.random.default_rng(42)
    n, d, scale = 50, 128, 0.2
    q, k, _ = _rand_head(rng, n, d)
    for signs in (None, rng.choice([-1.0, 1.0], size=d)):
        exact = scale * (q @ k.T)
        got = F.fp8_scores(q, k, scale, signs)
        if signs is None:
            qt, kt, rescale = q, k, 1.0
        else:
            m = signs[:, None] * F.hadamard(d)
            qt, kt, rescale = q @ m, k @ m, 1.0 / d
        _, a = F.quantize_rows(qt)
        _, b = F.quantize_tiles(kt)
        sub_q, sub_k = a * 2.0 ** -10, b * 2.0 ** -10
        bound = scale * rescale * (
            (np.abs(qt) @ np.abs(kt).T) * (2.0 ** -3 + 2.0 ** -8)
            + sub_q[:, None] * np.abs(kt).sum(axis=1)[None, :] * 1.07
            + np.abs(qt).sum(axis=1)[:, None] * sub_k[None, :] * 1.07
            + d * sub_q[:, None] * sub_k[None, :])
        assert np.all(np.abs(got - exact) <= bound), f"fp8 score error bound signs={signs is not None}"


def pin_fp8_incoherence_lowers_error():
    """The pages' claim for incoherent processing: with outlier channels the
    rotated FP8 scores err less than plain FP8 ones (the page reports 2.6x
    lower error for FlashAttention-3; here at least 1.5x on the scores)."""
    rng = np.random.default_rng(43)
    n, d, scale = 256, 128, 128 ** -0.5
    q, k, _ = _rand_head(rng, n, d)
    outliers = rng.choice(d, size=4, replace=False)
    q[:, outliers] *= 30.0
    k[:, outliers] *= 30.0
    signs = rng.choice([-1.0, 1.0], size=d)
    exact = scale * (q @ k.T)
    err_plain = np.linalg.norm(F.fp8_scores(q, k, scale, None) - exact)
    err_rot = np.linalg.norm(F.fp8_scores(q, k, scale, signs) - exact)
    assert err_plain > 1.5 * err_rot, f"plain {err_plain} vs incoherent {err_rot}"


ALL_PINS = [pin_golden_forward, pin_golden_backward, pin_vs_torch_sdpa,
            pin_backward_vs_autograd, pin_finite_differences, pin_brute_force,
            pin_online_recurrence, pin_forward_invariants, pin_backward_invariants,
            pin_gqa_vs_autograd, pin_gqa_finite_differences, pin_window_special_cases,
            pin_window_vs_torch, pin_window_brute_force, pin_block_mask_all_ones,
            pin_block_mask_vs_torch, pin_block_mask_brute_force, pin_block_mask_empty_rows,
            pin_block_diagonal_segments, pin_row_chunks_vs_torch, pin_row_chunks_zero_queries,
            pin_fp8_e4m3_golden,
            pin_fp8_e4m3_grid, pin_fp8_scales, pin_fp8_v_blocks, pin_fp8_forward_golden,
            pin_fp8_pv_error_bound, pin_fp8_hadamard, pin_fp8_rotation_is_exact, pin_fp8_error_bound,
            pin_fp8_incoherence_lowers_error]
