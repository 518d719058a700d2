"""Property-based checks of the fp64 oracle (hypothesis, CPU only).

The pins in oracle_pins.py check each identity on fixed shapes and seeds;
these draw the shapes, scales, masks, split points and head groupings at
random and check the same mathematics again over many cases:

* softmax rows: every row with a visible key sums to 1, and no probability
  lies outside the row's window (the definition of the masked softmax);
* the split-and-merge identity of the decomposed softmax (unite.ai page,
  softmax decomposition and merge), over random disjoint key subsets;
* invariances the definition fixes: shifting every key by one vector leaves
  O unchanged and moves lse by scale * q.c; folding the scale into Q; joint
  permutation of K and V rows (no mask); permutation of Q rows (no mask);
* window special cases: bounds of N-1 or more equal no bound, (-1, 0) is
  the causal mask, (0, 0) returns V row by row;
* backward identities: the key gradients sum to zero and the value
  gradients sum to the dO of the rows that see a key (each row of P sums to
  1 or is empty), for any mask; dQ against central finite differences of
  sum(dO * O);
* grouped K/V heads: the batched oracle with fewer K/V heads equals the one
  with every K/V head copied to its query heads, and its K/V gradients are
  the sums over those copies.

Each property is a plain function of its parameters; the hypothesis tests
draw the parameters, and test_properties_catch_planted_mistakes runs every
property on a fixed sample with a mistake planted in the oracle (the
mutations of test_oracle_mutations.py that these properties can reach) and
requires that one of them fails.
"""
import numpy as np
import pytest

pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import oracle.attention as A  # noqa: E402


def _arrays(seed, n, d, nk=None, spread=1.0):
    rng = np.random.default_rng(seed)
    nk = n if nk is None else nk
    q = rng.standard_normal((n, d)) * spread
    k = rng.standard_normal((nk, d))
    v = rng.standard_normal((nk, d))
    return rng, q, k, v


def _visible(i, j, mask):
    left, right = A.window_bounds(mask)
    return (left < 0 or j >= i - left) and (right < 0 or j <= i + right)


# ---------------------------------------------------------------- properties

def prop_rows_sum_to_one_inside_the_window(seed, n, d, scale, mask):
    _, q, k, _ = _arrays(seed, n, d, spread=2.0)
    p = A.probabilities_head(q, k, scale, mask)
    for i in range(n):
        vis = np.array([_visible(i, j, mask) for j in range(n)])
        assert np.all(p[i, ~vis] == 0.0)
        if vis.any():
            assert abs(p[i].sum() - 1.0) < 1e-12
        else:
            assert np.all(p[i] == 0.0)


def prop_merge_of_disjoint_key_sets(seed, n, nk, d, scale):
    rng, q, k, v = _arrays(seed, n, d, nk=nk, spread=3.0)
    split = 1 + int(rng.integers(nk - 1))
    perm = rng.permutation(nk)
    a, b = perm[:split], perm[split:]
    o, lse = A.forward_head(q, k, v, scale, False)
    o1, l1 = A.forward_head(q, k[a], v[a], scale, False)
    o2, l2 = A.forward_head(q, k[b], v[b], scale, False)
    om, lm = A.merge(o1, l1, o2, l2)
    np.testing.assert_allclose(om, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lse, rtol=1e-13, atol=1e-12)


def prop_key_shift_and_scale_folding(seed, n, d, scale, mask):
    rng, q, k, v = _arrays(seed, n, d, spread=2.0)
    o, lse = A.forward_head(q, k, v, scale, mask)
    c = rng.standard_normal(d)
    o_s, lse_s = A.forward_head(q, k + c, v, scale, mask)
    np.testing.assert_allclose(o_s, o, rtol=0, atol=1e-11)
    fin = np.isfinite(lse)
    assert np.array_equal(np.isfinite(lse_s), fin)
    np.testing.assert_allclose(lse_s[fin], (lse + scale * (q @ c))[fin], rtol=0, atol=1e-10)
    a = float(rng.uniform(0.25, 4.0))
    o_a, lse_a = A.forward_head(q * a, k, v, scale / a, mask)
    np.testing.assert_allclose(o_a, o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse_a[fin], lse[fin], rtol=0, atol=1e-11)


def prop_permutations_without_a_mask(seed, n, d, scale):
    rng, q, k, v = _arrays(seed, n, d)
    o, lse = A.forward_head(q, k, v, scale, False)
    pk = rng.permutation(n)
    o_k, lse_k = A.forward_head(q, k[pk], v[pk], scale, False)
    np.testing.assert_allclose(o_k, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_k, lse, rtol=0, atol=1e-12)
    pq = rng.permutation(n)
    o_q, lse_q = A.forward_head(q[pq], k, v, scale, False)
    np.testing.assert_allclose(o_q, o[pq], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_q, lse[pq], rtol=0, atol=1e-13)


def prop_window_special_cases(seed, n, d, scale, extra):
    _, q, k, v = _arrays(seed, n, d, spread=2.0)
    wide = n - 1 + extra
    o_n, l_n = A.forward_head(q, k, v, scale, False)
    for mask in ((wide, wide), (-1, wide), (wide, -1), (-1, -1)):
        o_w, l_w = A.forward_head(q, k, v, scale, mask)
        assert np.array_equal(o_w, o_n) and np.array_equal(l_w, l_n), mask
    o_c, l_c = A.forward_head(q, k, v, scale, True)
    for mask in ((-1, 0), (wide, 0)):
        o_w, l_w = A.forward_head(q, k, v, scale, mask)
        assert np.array_equal(o_w, o_c) and np.array_equal(l_w, l_c), mask
    # (0, 0): each row sees only its own key
    o_0, l_0 = A.forward_head(q, k, v, scale, (0, 0))
    np.testing.assert_array_equal(o_0, v)
    np.testing.assert_allclose(l_0, scale * np.sum(q * k, axis=1), rtol=0, atol=1e-12)


def prop_backward_sums(seed, n, d, scale, mask):
    rng, q, k, v = _arrays(seed, n, d)
    do = rng.standard_normal((n, d))
    _, dk, dv = A.backward_head(q, k, v, do, scale, mask)
    np.testing.assert_allclose(dk.sum(axis=0), np.zeros(d), rtol=0, atol=1e-11)
    rows_with_keys = np.array([any(_visible(i, j, mask) for j in range(n)) for i in range(n)])
    np.testing.assert_allclose(dv.sum(axis=0), do[rows_with_keys].sum(axis=0), rtol=0,
                               atol=1e-11)


def prop_dq_against_finite_differences(seed, n, d, scale, mask):
    rng, q, k, v = _arrays(seed, n, d)
    do = rng.standard_normal((n, d))
    dq, _, _ = A.backward_head(q, k, v, do, scale, mask)

    def f(qq):
        return float(np.sum(do * A.forward_head(qq, k, v, scale, mask)[0]))

    h = 1e-6
    num = np.zeros_like(q)
    for i in range(n):
        for j in range(d):
            e = np.zeros_like(q)
            e[i, j] = h
            num[i, j] = (f(q + e) - f(q - e)) / (2 * h)
    np.testing.assert_allclose(dq, num, rtol=0, atol=1e-7)


def prop_grouped_heads_equal_copied_heads(seed, n, d, groups, mask):
    heads, kv_heads = groups
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, heads, n, d))
    k = rng.standard_normal((1, kv_heads, n, d))
    v = rng.standard_normal((1, kv_heads, n, d))
    do = rng.standard_normal((1, heads, n, d))
    rep = heads // kv_heads
    k_full, v_full = np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1)
    o, lse = A.forward(q, k, v, 0.5, mask)
    o_f, lse_f = A.forward(q, k_full, v_full, 0.5, mask)
    assert np.array_equal(o, o_f) and np.array_equal(lse, lse_f)
    dq, dk, dv = A.backward(q, k, v, do, 0.5, mask)
    dq_f, dk_f, dv_f = A.backward(q, k_full, v_full, do, 0.5, mask)
    assert np.array_equal(dq, dq_f)
    np.testing.assert_allclose(dk, dk_f.reshape(1, kv_heads, rep, n, d).sum(axis=2), rtol=0,
                               atol=1e-12)
    np.testing.assert_allclose(dv, dv_f.reshape(1, kv_heads, rep, n, d).sum(axis=2), rtol=0,
                               atol=1e-12)


# ---------------------------------------------------------------- hypothesis

def _settings(n):
    return settings(max_examples=n, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


seeds = st.integers(0, 2**31 - 1)
scales = st.floats(0.05, 2.0)
masks = st.one_of(st.booleans(), st.tuples(st.integers(-1, 12), st.integers(-1, 12)))
groupings = st.sampled_from([(2, 1), (4, 2), (6, 3), (3, 3), (4, 1)])


@_settings(150)
@given(seed=seeds, n=st.integers(1, 24), d=st.integers(1, 8), scale=scales, mask=masks)
def test_rows_sum_to_one_inside_the_window(seed, n, d, scale, mask):
    prop_rows_sum_to_one_inside_the_window(seed, n, d, scale, mask)


@_settings(150)
@given(seed=seeds, n=st.integers(1, 20), nk=st.integers(2, 30), d=st.integers(1, 8),
       scale=scales)
def test_merge_of_disjoint_key_sets(seed, n, nk, d, scale):
    prop_merge_of_disjoint_key_sets(seed, n, nk, d, scale)


@_settings(150)
@given(seed=seeds, n=st.integers(1, 20), d=st.integers(1, 8), scale=scales, mask=masks)
def test_key_shift_and_scale_folding(seed, n, d, scale, mask):
    prop_key_shift_and_scale_folding(seed, n, d, scale, mask)


@_settings(150)
@given(seed=seeds, n=st.integers(2, 20), d=st.integers(1, 8), scale=scales)
def test_permutations_without_a_mask(seed, n, d, scale):
    prop_permutations_without_a_mask(seed, n, d, scale)


@_settings(150)
@given(seed=seeds, n=st.integers(1, 20), d=st.integers(1, 8), scale=scales,
       extra=st.integers(0, 5))
def test_window_special_cases(seed, n, d, scale, extra):
    prop_window_special_cases(seed, n, d, scale, extra)


@_settings(150)
@given(seed=seeds, n=st.integers(1, 16), d=st.integers(1, 6), scale=st.floats(0.05, 1.5),
       mask=masks)
def test_backward_sums(seed, n, d, scale, mask):
    prop_backward_sums(seed, n, d, scale, mask)


@_settings(40)
@given(seed=seeds, n=st.integers(1, 8), d=st.integers(1, 4), scale=st.floats(0.1, 1.0),
       mask=masks)
def test_dq_against_finite_differences(seed, n, d, scale, mask):
    prop_dq_against_finite_differences(seed, n, d, scale, mask)


@_settings(60)
@given(seed=seeds, n=st.integers(1, 10), d=st.integers(1, 6), groups=groupings, mask=masks)
def test_grouped_heads_equal_copied_heads(seed, n, d, groups, mask):
    prop_grouped_heads_equal_copied_heads(seed, n, d, groups, mask)


# ---------------------------------------------------------------- planted mistakes

def _sample_runs(rng):
    """Each property on a few fixed parameter sets (masks: none, causal, two windows)."""
    runs = []
    for mask in (False, True, (3, 1), (0, 4)):
        seed = int(rng.integers(2**31))
        runs += [
            (prop_rows_sum_to_one_inside_the_window, (seed, 9, 4, 0.7, mask)),
            (prop_key_shift_and_scale_folding, (seed, 9, 4, 0.7, mask)),
            (prop_backward_sums, (seed, 7, 3, 0.6, mask)),
            (prop_dq_against_finite_differences, (seed, 5, 3, 0.6, mask)),
            (prop_grouped_heads_equal_copied_heads, (seed, 6, 3, (4, 2), mask)),
        ]
    seed = int(rng.integers(2**31))
    runs += [
        (prop_merge_of_disjoint_key_sets, (seed, 7, 11, 4, 0.8)),
        (prop_permutations_without_a_mask, (seed, 9, 4, 0.7)),
        (prop_window_special_cases, (seed, 9, 4, 0.7, 2)),
    ]
    return runs


# the mutations of test_oracle_mutations.py these properties can reach. Out of
# reach: block masks and row chunks past 512 rows (not exercised here); a
# negated dK (its sum stays zero, and no property compares dK with another
# value); a reversed head map (it agrees with copying the K/V heads in the
# same reversed order). The pins against torch catch those.
REACHABLE = ["scale_dropped", "causal_mask_flipped", "causal_mask_excludes_diagonal", "lse_base2",
             "lse_drops_sum", "bwd_drops_D", "bwd_dq_transposed", "bwd_dv_untransposed",
             "bwd_dq_scale_dropped", "fwd_p_transposed", "gqa_head_map_modulo",
             "gqa_grads_overwritten", "window_left_bound_strict", "window_bounds_swapped",
             "window_right_bound_one_wide"]


def test_properties_pass_on_the_sample():
    for prop, args in _sample_runs(np.random.default_rng(5)):
        prop(*args)


@pytest.mark.parametrize("name", REACHABLE)
def test_properties_catch_planted_mistakes(name, monkeypatch):
    import test_oracle_mutations as M
    attr, fn = M.MUTATIONS[name]
    A._ORIG = {a: getattr(A, a) for a in ("_scores", "_row_softmax_stats", "forward_head",
                                          "backward_head", "backward", "kv_head")}
    monkeypatch.setattr(A, attr, fn)
    failed = []
    for prop, args in _sample_runs(np.random.default_rng(5)):
        try:
            with np.errstate(all="ignore"):
                prop(*args)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(prop.__name__)
    assert failed, f"no property caught the planted mistake {name}"
