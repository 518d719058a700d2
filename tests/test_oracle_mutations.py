"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.

Each mutation replaces one oracle function with a copy that carries one
mistake: a dropped term, a wrong sign or index, a transposed operand, a wrong
log base, a flipped mask. The pins must reject every one of them.
"""
import numpy as np
import pytest

import oracle.attention as A
from oracle_pins import ALL_PINS


def _scores_no_scale(q_rows, k, scale, row_ids, causal):
    return A._ORIG["_scores"](q_rows, k, 1.0, row_ids, causal)


def _scores_flipped_mask(q_rows, k, scale, row_ids, causal):
    s = scale * (q_rows @ k.T)
    if causal:
        keys = np.arange(k.shape[0])[None, :]
        s = np.where(keys >= row_ids[:, None], s, -np.inf)
    return s


def _scores_strict_mask(q_rows, k, scale, row_ids, causal):
    s = scale * (q_rows @ k.T)
    if causal:
        keys = np.arange(k.shape[0])[None, :]
        s = np.where(keys < row_ids[:, None] + (row_ids[:, None] == 0), s, -np.inf)
    return s


def _stats_log2(s):
    return A._ORIG["_row_softmax_stats"](s) / np.log(2.0)


def _stats_no_max(s):
    with np.errstate(over="ignore", divide="ignore"):
        return np.log(np.sum(np.exp(s), axis=1))


def _stats_max_only(s):
    return np.max(s, axis=1) + np.log(s.shape[1])


def _bwd_variant(kind):
    def bwd(q, k, v, do, scale, causal):
        p = A.probabilities_head(q, k, scale, causal)
        o = p @ v
        d_row = np.sum(do * o, axis=1)
        dp = do @ v.T
        ds = p * (dp - d_row[:, None]) if kind != "drop_D" else p * dp
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        dv = p.T @ do
        if kind == "sign_dk":
            dk = -dk
        if kind == "transpose_dq":
            dq = scale * (ds.T @ k) if ds.shape[0] == ds.shape[1] else dq * 1.01
        if kind == "dv_no_transpose":
            dv = p @ do
        if kind == "dq_no_scale":
            dq = ds @ k
        return dq, dk, dv
    return bwd


def _fwd_transposed_p(q, k, v, scale, causal, rows=None):
    p = A.probabilities_head(q, k, scale, causal)
    o = p.T @ v
    ids = np.arange(q.shape[0]) if rows is None else rows
    lse = A._ORIG["forward_head"](q, k, v, scale, causal, rows)[1]
    return o[ids], lse


def _kv_head_modulo(h, heads, kv_heads):
    return h % kv_heads


def _kv_head_reversed(h, heads, kv_heads):
    return (heads - 1 - h) // (heads // kv_heads)


def _backward_not_summed(q, k, v, do, scale, causal):
    heads, kv_heads = q.shape[1], k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros(np.shape(k))
    dv = np.zeros(np.shape(v))
    for b in range(q.shape[0]):
        for h in range(heads):
            g = A.kv_head(h, heads, kv_heads)
            dq[b, h], dk[b, g], dv[b, g] = A.backward_head(q[b, h], k[b, g], v[b, g], do[b, h],
                                                        scale, causal)
    return dq, dk, dv


def _window_variant(kind):
    def scores(q_rows, k, scale, row_ids, causal):
        s = scale * (q_rows @ k.T)
        left, right = A.window_bounds(causal)
        if kind == "swapped":
            left, right = right, left
        keys = np.arange(k.shape[0])[None, :]
        rows = row_ids[:, None]
        if left >= 0:
            lo = rows - left + (1 if kind == "left_strict" else 0)
            s = np.where(keys >= lo, s, -np.inf)
        if right >= 0:
            hi = rows + right + (1 if kind == "right_wide" else 0)
            s = np.where(keys <= hi, s, -np.inf)
        return s
    return scores


MUTATIONS = {
    "scale_dropped": ("_scores", _scores_no_scale),
    "causal_mask_flipped": ("_scores", _scores_flipped_mask),
    "causal_mask_excludes_diagonal": ("_scores", _scores_strict_mask),
    "lse_base2": ("_row_softmax_stats", _stats_log2),
    "softmax_without_max": ("_row_softmax_stats", _stats_no_max),
    "lse_drops_sum": ("_row_softmax_stats", _stats_max_only),
    "bwd_drops_D": ("backward_head", _bwd_variant("drop_D")),
    "bwd_dk_sign": ("backward_head", _bwd_variant("sign_dk")),
    "bwd_dq_transposed": ("backward_head", _bwd_variant("transpose_dq")),
    "bwd_dv_untransposed": ("backward_head", _bwd_variant("dv_no_transpose")),
    "bwd_dq_scale_dropped": ("backward_head", _bwd_variant("dq_no_scale")),
    "fwd_p_transposed": ("forward_head", _fwd_transposed_p),
    "gqa_head_map_modulo": ("kv_head", _kv_head_modulo),
    "gqa_head_map_reversed": ("kv_head", _kv_head_reversed),
    "gqa_grads_overwritten": ("backward", _backward_not_summed),
    "window_left_bound_strict": ("_scores", _window_variant("left_strict")),
    "window_bounds_swapped": ("_scores", _window_variant("swapped")),
    "window_right_bound_one_wide": ("_scores", _window_variant("right_wide")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    A._ORIG = {a: getattr(A, a) for a in ("_scores", "_row_softmax_stats", "forward_head",
                                          "backward_head", "backward", "kv_head")}
    monkeypatch.setattr(A, attr, fn)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
