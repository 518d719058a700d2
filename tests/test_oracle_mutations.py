"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.

Each mutation replaces one oracle function with a copy that carries one
mistake: a dropped term, a wrong sign or index, a transposed operand, a wrong
log base, a flipped mask. The pins must reject every one of them.
"""
import numpy as np
import pytest

import oracle.attention as A
import oracle.fp8 as F
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
    def bwd(q, k, v, do, scale, causal, block_mask=None):
        p = A.probabilities_head(q, k, scale, causal, block_mask)
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


def _fwd_transposed_p(q, k, v, scale, causal, rows=None, block_mask=None):
    p = A.probabilities_head(q, k, scale, causal, block_mask)
    o = p.T @ v
    ids = np.arange(q.shape[0]) if rows is None else rows
    lse = A._ORIG["forward_head"](q, k, v, scale, causal, rows, block_mask=block_mask)[1]
    return o[ids], lse


def _fwd_chunk_variant(kind):
    """forward_head with the row chunks or the row subset mishandled."""
    def fwd(q, k, v, scale, causal, rows=None, block_mask=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
        if kind == "rows_ignored":
            rows = np.arange(rows.shape[0])
        out = np.zeros((rows.shape[0], v.shape[1]))
        lse = np.zeros(rows.shape[0])
        for start in range(0, rows.shape[0], A._ROW_CHUNK):
            ids = rows[start:start + A._ROW_CHUNK]
            # the mistake: row ids counted from the start of the chunk
            mask_ids = ids - start if kind == "chunk_local_ids" else ids
            s = A._apply_block_mask(A._scores(q[ids], k, scale, mask_ids, causal), mask_ids,
                                    block_mask)
            l_rows = A._row_softmax_stats(s)
            p = np.exp(s - np.where(np.isfinite(l_rows), l_rows, 0.0)[:, None])
            p = np.where(np.isfinite(l_rows)[:, None], p, 0.0)
            out[start:start + ids.shape[0]] = p @ v
            lse[start:start + ids.shape[0]] = l_rows
        return out, lse
    return fwd


def _kv_head_modulo(h, heads, kv_heads):
    return h % kv_heads


def _kv_head_reversed(h, heads, kv_heads):
    return (heads - 1 - h) // (heads // kv_heads)


def _backward_not_summed(q, k, v, do, scale, causal, block_mask=None):
    heads, kv_heads = q.shape[1], k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros(np.shape(k))
    dv = np.zeros(np.shape(v))
    for b in range(q.shape[0]):
        for h in range(heads):
            g = A.kv_head(h, heads, kv_heads)
            dq[b, h], dk[b, g], dv[b, g] = A.backward_head(q[b, h], k[b, g], v[b, g], do[b, h],
                                                        scale, causal,
                                                        block_mask=A._head_mask(block_mask, b, h))
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


def _block_mask_variant(kind):
    def apply(s, row_ids, block_mask):
        if block_mask is None or kind == "ignored":
            return s
        size = 64 if kind == "size_64" else 128
        bm = np.asarray(block_mask) != 0
        rb = (np.asarray(row_ids) // size)[:, None]
        kb = (np.arange(s.shape[1]) // size)[None, :]
        if kind == "size_64":
            rb, kb = np.minimum(rb, bm.shape[0] - 1), np.minimum(kb, bm.shape[1] - 1)
        keep = bm[kb, rb] if kind == "transposed" else bm[rb, kb]
        return np.where(keep, s, -np.inf)
    return apply


def _probabilities_empty_rows_kept(q, k, scale, causal, block_mask=None):
    ids = np.arange(q.shape[0])
    s = A._apply_block_mask(A._scores(q, k, scale, ids, causal), ids, block_mask)
    lse = A._row_softmax_stats(s)
    return np.exp(s - lse[:, None])


def _e4m3_variant(kind):
    def rnd(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x) if kind == "no_saturation" else np.minimum(np.abs(x), F.E4M3_MAX)
        _, k = np.frexp(np.where(a > 0, a, 1.0))
        e = k - 1.0 if kind == "flush_subnormals" else np.maximum(k - 1.0, -6.0)
        step = np.exp2(e - (2.0 if kind == "two_mantissa_bits" else 3.0))
        if kind == "ties_away":
            q = np.floor(a / step + 0.5) * step
        else:
            q = np.round(a / step) * step
        if kind == "flush_subnormals":
            q = np.where(a < 2.0 ** -6, 0.0, q)
        if kind != "no_saturation":
            q = np.minimum(q, F.E4M3_MAX)
        return np.where(x < 0, -q, q)
    return rnd


def _hadamard_wrong_block(d):
    h = F._ORIG["hadamard"](d)
    if d >= 2:
        h[d // 2:, d // 2:] *= -1.0   # [[H, H], [H, H]]: no longer orthogonal
    return h


def _scale_floor(maxabs):
    maxabs = np.asarray(maxabs, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(maxabs > 0, maxabs, F.E4M3_MAX) / F.E4M3_MAX))
    return np.exp2(e)


def _tiles_per_row(x, tile=F.KEY_TILE):
    return F.quantize_rows(x)


def _scores_variant(kind):
    def scores(q, k, scale, signs=None, quantize=True):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        d = q.shape[1]
        rescale = 1.0
        if signs is not None:
            m = np.asarray(signs, dtype=np.float64)[:, None] * F.hadamard(d)
            if kind == "rotate_q_only":
                q, rescale = q @ m, 1.0 / d
            else:
                q, k = q @ m, k @ m
                rescale = 1.0 if kind == "no_rescale" else 1.0 / d
        if not quantize:
            return scale * rescale * (q @ k.T)
        q8, a = F.quantize_rows(q)
        k8, b = F.quantize_tiles(k)
        if kind == "k_scale_dropped":
            b = np.ones_like(b)
        return scale * rescale * (a[:, None] * (q8 @ k8.T) * b[None, :])
    return scores


def _fp8_forward_variant(kind):
    def fwd(q, k, v, scale, causal, signs=None, quantize=True):
        s = F.fp8_scores(q, k, scale, signs, quantize)
        n = s.shape[0]
        if causal:
            s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
        lse = A._row_softmax_stats(s)
        v = np.asarray(v, dtype=np.float64)
        if not quantize:
            return np.exp(s - lse[:, None]) @ v, lse
        if kind == "exact_max_reference":
            p = np.exp(s - np.max(s, axis=1, keepdims=True))
        else:
            m = np.ceil(np.max(s, axis=1, keepdims=True) / np.log(2.0))
            p = np.exp2(s / np.log(2.0) - m)
        v8, vs = F.quantize_key_blocks(v)
        if kind == "p_unrounded":
            pq = p
        elif kind == "p_unscaled":
            pq = F.e4m3_round(p)
        else:
            pq = F.e4m3_round(p * 256.0) / 256.0
        vq = v if kind == "v_unrounded" else v8 * vs
        den = np.sum(pq if kind == "sum_of_rounded" else p, axis=1, keepdims=True)
        return (pq @ vq) / den, lse
    return fwd


def _v_blocks_of_64(x, block=F.V_BLOCK):
    return F._ORIG["quantize_key_blocks"](x, 64)


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
    "fwd_chunk_local_row_ids": ("forward_head", _fwd_chunk_variant("chunk_local_ids")),
    "fwd_rows_argument_ignored": ("forward_head", _fwd_chunk_variant("rows_ignored")),
    "gqa_head_map_modulo": ("kv_head", _kv_head_modulo),
    "gqa_head_map_reversed": ("kv_head", _kv_head_reversed),
    "gqa_grads_overwritten": ("backward", _backward_not_summed),
    "window_left_bound_strict": ("_scores", _window_variant("left_strict")),
    "window_bounds_swapped": ("_scores", _window_variant("swapped")),
    "window_right_bound_one_wide": ("_scores", _window_variant("right_wide")),
    "block_mask_transposed": ("_apply_block_mask", _block_mask_variant("transposed")),
    "block_mask_blocks_of_64": ("_apply_block_mask", _block_mask_variant("size_64")),
    "block_mask_ignored": ("_apply_block_mask", _block_mask_variant("ignored")),
    "block_mask_empty_rows_not_zeroed": ("probabilities_head", _probabilities_empty_rows_kept),
}
FP8_MUTATIONS = {
    "e4m3_two_mantissa_bits": ("e4m3_round", _e4m3_variant("two_mantissa_bits")),
    "e4m3_ties_away_from_zero": ("e4m3_round", _e4m3_variant("ties_away")),
    "e4m3_flushes_subnormals": ("e4m3_round", _e4m3_variant("flush_subnormals")),
    "e4m3_no_saturation": ("e4m3_round", _e4m3_variant("no_saturation")),
    "hadamard_wrong_block": ("hadamard", _hadamard_wrong_block),
    "fp8_scale_rounds_down": ("pow2_scale", _scale_floor),
    "fp8_k_scale_per_row": ("quantize_tiles", _tiles_per_row),
    "fp8_rotation_not_rescaled": ("fp8_scores", _scores_variant("no_rescale")),
    "fp8_only_q_rotated": ("fp8_scores", _scores_variant("rotate_q_only")),
    "fp8_k_scale_dropped": ("fp8_scores", _scores_variant("k_scale_dropped")),
    "fp8_p_not_rounded": ("forward_fp8_head", _fp8_forward_variant("p_unrounded")),
    "fp8_v_not_rounded": ("forward_fp8_head", _fp8_forward_variant("v_unrounded")),
    "fp8_row_sum_of_rounded_p": ("forward_fp8_head", _fp8_forward_variant("sum_of_rounded")),
    "fp8_v_blocks_of_64": ("quantize_key_blocks", _v_blocks_of_64),
    "fp8_p_rounded_without_scale": ("forward_fp8_head", _fp8_forward_variant("p_unscaled")),
    "fp8_p_reference_exact_max": ("forward_fp8_head", _fp8_forward_variant("exact_max_reference")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS) + sorted(FP8_MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    module, (attr, fn) = (A, MUTATIONS[name]) if name in MUTATIONS else (F, FP8_MUTATIONS[name])
    A._ORIG = {a: getattr(A, a) for a in ("_scores", "_row_softmax_stats", "forward_head",
                                          "backward_head", "backward", "kv_head")}
    F._ORIG = {"hadamard": F.hadamard, "quantize_key_blocks": F.quantize_key_blocks}
    monkeypatch.setattr(module, attr, fn)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
