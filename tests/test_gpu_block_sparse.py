"""GPU parity of block-sparse attention through the C ABI against the fp64
oracle: blocks of 128 query rows x 128 keys whose mask byte is 0 are masked,
on top of the window mask; a row that sees no key has O = 0, lse = -inf and
no gradient."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_14_amd import (fa_backward_block_sparse, fa_backward_gqa,
                                   fa_backward_grads_block_sparse, fa_backward_prep,
                                   fa_backward_window, fa_forward_block_sparse, fa_forward_gqa,
                                   fa_forward_window)
from exact_io_aware_14_amd.inputs import (BLOCK_SPARSE_WORKLOADS, draw, draw_block_mask,
                                          draw_segments, to_f64, workload_block_mask)
from parity import (LSE_MAX_ABS, check_grad, check_o, dq_allowance, dq_allowances, log, metrics,
                    sample_heads)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (B, H, H_kv, N, d): ragged lengths, grouped heads, the three head dimensions
SHAPES = [(1, 2, 2, 300, 64), (1, 4, 2, 513, 128), (2, 2, 1, 200, 256), (1, 2, 1, 700, 128)]
# no window, causal, a causal window crossing blocks, both sides bounded
WINDOWS = [(-1, -1), (-1, 0), (150, 0), (40, 200)]
# random half-dense masks with the diagonal kept; without it and with whole
# block rows zeroed (rows that see nothing); packed segments
PATTERNS = ["diag", "empty", "segments"]


def _mask(pattern, B, H, N, seed):
    if pattern == "diag":
        return draw_block_mask(N, seed, 0.5, heads=(B, H))
    if pattern == "empty":
        return draw_block_mask(N, seed, 0.5, heads=(B, H), diagonal=False, empty_rows=1)
    return draw_segments(N, seed, heads=(B, H))


def check_lse_masked(lse, ref, what):
    """lse against the oracle where a row sees a key; -inf exactly where it
    sees none."""
    assert not np.any(np.isnan(lse)), f"{what}: NaN in lse"
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    assert np.all(np.isfinite(lse[~empty])), f"{what}: non-finite lse"
    max_abs, _ = metrics(lse[~empty], ref[~empty])
    log(f"  {what}: lse max_abs={max_abs:.3e} empty rows={int(empty.sum())}")
    assert max_abs <= LSE_MAX_ABS, (what, max_abs)


def _ids(cases):
    return [f"{w[0]},{w[1]}" for w in cases]


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("window", WINDOWS, ids=_ids(WINDOWS))
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_block_sparse_forward(shape, window, pattern):
    B, H, Hkv, N, d = shape
    q, k, v = draw((B, H, N, d), 700 + N, kv_heads=Hkv)
    bm = _mask(pattern, B, H, N, 710 + N)
    scale = 1.0 / math.sqrt(d)
    log(f"case block-sparse forward {shape} {window} {pattern}")
    o, lse = fa_forward_block_sparse(q.to(DEV), k.to(DEV), v.to(DEV), bm.to(DEV), *window,
                                     scale=scale)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for h in range(H):
            g = oracle.kv_head(h, H, Hkv)
            ro, rl = oracle.forward_head(to_f64(q[b, h]), to_f64(k[b, g]), to_f64(v[b, g]),
                                         scale, window, block_mask=bm[b, h].numpy())
            what = f"{shape} {window} {pattern} b={b} h={h}"
            empty = np.isneginf(rl)
            assert np.all(o[b, h][empty] == 0.0), f"{what}: O of empty rows"
            check_o(o[b, h], ro, what)
            check_lse_masked(lse[b, h], rl, what)


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("window", WINDOWS, ids=_ids(WINDOWS))
@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_block_sparse_backward(shape, window, pattern):
    B, H, Hkv, N, d = shape
    q, k, v, do = draw((B, H, N, d), 800 + N, with_grad=True, kv_heads=Hkv)
    bm = _mask(pattern, B, H, N, 810 + N)
    scale = 1.0 / math.sqrt(d)
    log(f"case block-sparse backward {shape} {window} {pattern}")
    qd, kd, vd, dod, bmd = (x.to(DEV) for x in (q, k, v, do, bm))
    o, lse = fa_forward_block_sparse(qd, kd, vd, bmd, *window, scale=scale)
    dq, dk, dv = fa_backward_block_sparse(qd, kd, vd, o, dod, lse, bmd, *window, scale=scale)
    torch.cuda.synchronize()
    args = (to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, window)
    rq, rk, rv = oracle.backward(*args, block_mask=bm.numpy())
    aq = dq_allowances(*args, block_mask=bm.numpy())
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    for b in range(B):
        for h in range(H):
            check_grad(dq[b, h], rq[b, h], f"{shape} {window} {pattern} b={b} h={h} dQ",
                       allow=aq[b, h])
        for g in range(Hkv):
            check_grad(dk[b, g], rk[b, g], f"{shape} {window} {pattern} b={b} kv={g} dK")
            check_grad(dv[b, g], rv[b, g], f"{shape} {window} {pattern} b={b} kv={g} dV")
    # rows that see no key have no gradient; keys no row sees neither
    for b in range(B):
        for h in range(H):
            empty = ~np.isfinite(lse[b, h].cpu().numpy())
            assert np.all(dq[b, h][empty] == 0.0)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_all_ones_mask_is_the_window_call(d):
    """A mask of ones changes nothing: bitwise the results of the _window
    calls (and, for no window, of the plain calls) on the same inputs."""
    B, H, Hkv, N = 1, 4, 2, 333
    q, k, v, do = (x.to(DEV) for x in draw((B, H, N, d), 90 + d, with_grad=True, kv_heads=Hkv))
    nb = (N + 127) // 128
    ones = torch.ones((nb, nb), dtype=torch.uint8, device=DEV)
    for window in ((-1, 0), (100, 3), (-1, -1)):
        log(f"case all-ones mask d={d} {window}")
        o1, l1 = fa_forward_block_sparse(q, k, v, ones, *window)
        g1 = fa_backward_block_sparse(q, k, v, o1, do, l1, ones, *window)
        if window == (-1, -1):
            o2, l2 = fa_forward_gqa(q, k, v, causal=False)
            g2 = fa_backward_gqa(q, k, v, o2, do, l2, causal=False)
        else:
            o2, l2 = fa_forward_window(q, k, v, *window)
            g2 = fa_backward_window(q, k, v, o2, do, l2, *window)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), window
        for a, b in zip(g1, g2):
            assert torch.equal(a, b), window


def test_zero_mask_and_shared_mask():
    """An all-zero mask: O = 0, lse = -inf and every gradient 0. A 2-D mask
    (head stride 0) gives the results of the same mask repeated per head."""
    B, H, Hkv, N, d = 2, 4, 2, 400, 128
    q, k, v, do = (x.to(DEV) for x in draw((B, H, N, d), 97, with_grad=True, kv_heads=Hkv))
    nb = (N + 127) // 128
    log("case zero mask")
    zero = torch.zeros((nb, nb), dtype=torch.uint8, device=DEV)
    o, lse = fa_forward_block_sparse(q, k, v, zero, -1, 0)
    grads = fa_backward_block_sparse(q, k, v, o, do, lse, zero, -1, 0)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    for g in grads:
        assert torch.all(g == 0)
    log("case shared mask")
    shared = draw_block_mask(N, 98, 0.5).to(DEV)
    per_head = shared.expand(B, H, nb, nb).contiguous()
    o1, l1 = fa_forward_block_sparse(q, k, v, shared, -1, 0)
    o2, l2 = fa_forward_block_sparse(q, k, v, per_head, -1, 0)
    g1 = fa_backward_block_sparse(q, k, v, o1, do, l1, shared, -1, 0)
    g2 = fa_backward_block_sparse(q, k, v, o2, do, l2, per_head, -1, 0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    # a bool mask is the same bytes
    o3, l3 = fa_forward_block_sparse(q, k, v, shared.bool(), -1, 0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_block_sparse_stages_match_backward():
    B, H, Hkv, N, d = 1, 4, 2, 600, 64
    q, k, v, do = (x.to(DEV) for x in draw((B, H, N, d), 99, with_grad=True, kv_heads=Hkv))
    bm = draw_block_mask(N, 100, 0.5, heads=(B, H), diagonal=False).to(DEV)
    log("case block-sparse stages")
    o, lse = fa_forward_block_sparse(q, k, v, bm, 300, 0)
    ref = fa_backward_block_sparse(q, k, v, o, do, lse, bm, 300, 0)
    ws = fa_backward_prep(o, do, lse)
    got = fa_backward_grads_block_sparse(q, k, v, do, lse, ws, bm, 300, 0)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_block_sparse_full_size_workload():
    """The block-sparse workload at full size: sampled heads of O and lse and
    one head's gradients against the oracle."""
    w = BLOCK_SPARSE_WORKLOADS[0]
    window = (-1, 0) if w.causal else (-1, -1)
    log(f"workload {w.name}")
    q, k, v, do = draw(w.shape, w.seed, with_grad=True)
    bm = workload_block_mask(w)
    qd, kd, vd, dod, bmd = (x.to(DEV) for x in (q, k, v, do, bm))
    o, lse = fa_forward_block_sparse(qd, kd, vd, bmd, *window, scale=w.scale)
    dq, dk, dv = fa_backward_block_sparse(qd, kd, vd, o, dod, lse, bmd, *window, scale=w.scale)
    torch.cuda.synchronize()
    for x in (o, dq, dk, dv, lse):
        assert torch.isfinite(x.float()).all()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    heads = sample_heads(w.B, w.H, 2, seed=w.seed)
    for b, h in heads:
        ro, rl = oracle.forward_head(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), w.scale,
                                     window, block_mask=bm[b, h].numpy())
        check_o(o[b, h], ro, f"{w.name} b={b} h={h}")
        check_lse_masked(lse[b, h], rl, f"{w.name} b={b} h={h}")
    b, h = heads[0]
    args = (to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), to_f64(do[b, h]), w.scale, window)
    rq, rk, rv = oracle.backward_head(*args, block_mask=bm[b, h].numpy())
    aq = dq_allowance(*args, block_mask=bm[b, h].numpy())
    for name, got, ref, al in (("dQ", dq, rq, aq), ("dK", dk, rk, None), ("dV", dv, rv, None)):
        check_grad(got[b, h].float().cpu().numpy(), ref, f"{w.name} b={b} h={h} {name}",
                   allow=al)


@pytest.mark.parametrize("d", [64, 256])
def test_block_sparse_long_rows_and_columns(d):
    """N = 8300: 65 mask blocks per row and column, so every walk reads its
    mask in two 64-block pieces. Sampled rows of O and lse of both heads
    and the gradients of the whole problem against the oracle, causal and a
    window."""
    B, H, Hkv, N = 1, 2, 1, 8300
    q, k, v, do = draw((B, H, N, d), 120 + d, with_grad=True, kv_heads=Hkv)
    bm = draw_block_mask(N, 121 + d, 0.3, heads=(B, H))
    bm[0, 1, :, 64] = 1  # the last block column, seen by every row of head 1
    scale = 1.0 / math.sqrt(d)
    rows = np.array(sorted(set(range(0, 200)) | set(range(8100, N)) |
                           set(np.random.default_rng(d).integers(0, N, 300).tolist())))
    qd, kd, vd, dod, bmd = (x.to(DEV) for x in (q, k, v, do, bm))
    for window in ((-1, 0), (3000, 100)):
        log(f"case block-sparse long d={d} {window}")
        o, lse = fa_forward_block_sparse(qd, kd, vd, bmd, *window, scale=scale)
        dq, dk, dv = fa_backward_block_sparse(qd, kd, vd, o, dod, lse, bmd, *window, scale=scale)
        torch.cuda.synchronize()
        on, ln = o.float().cpu().numpy(), lse.cpu().numpy()
        for h in range(H):
            ro, rl = oracle.forward_head(to_f64(q[0, h]), to_f64(k[0, 0]), to_f64(v[0, 0]), scale,
                                         window, rows=rows, block_mask=bm[0, h].numpy())
            check_o(on[0, h][rows], ro, f"long d={d} {window} h={h}")
            check_lse_masked(ln[0, h][rows], rl, f"long d={d} {window} h={h}")
        args = (to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, window)
        rq, rk, rv = oracle.backward(*args, block_mask=bm.numpy())
        aq = dq_allowances(*args, block_mask=bm.numpy())
        for name, got, ref, al in (("dQ", dq, rq, aq), ("dK", dk, rk, None),
                                   ("dV", dv, rv, None)):
            got = got.float().cpu().numpy()
            for h in range(got.shape[1]):
                check_grad(got[0, h], ref[0, h], f"long d={d} {window} h={h} {name}",
                           allow=None if al is None else al[0, h])


def test_block_sparse_graph_replays_match_eager():
    """Block-sparse calls captured into a HIP graph replay like eager calls,
    also with new mask contents written between replays (the kernels read
    the mask at run time)."""
    shape = (1, 4, 600, 128)
    B, H, N, d = shape
    nb = (N + 127) // 128
    q, k, v, do = (torch.empty(shape, dtype=torch.bfloat16, device=DEV) for _ in range(4))
    bm = torch.empty((B, H, nb, nb), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    from exact_io_aware_14_amd import fa_backward_workspace_size
    ws = torch.empty(fa_backward_workspace_size(*shape), dtype=torch.uint8, device=DEV)

    def step():
        fa_forward_block_sparse(q, k, v, bm, -1, 0, o=o, lse=lse)
        fa_backward_block_sparse(q, k, v, o, do, lse, bm, -1, 0, dq=dq, dk=dk, dv=dv,
                                 workspace=ws)

    for x, y in zip((q, k, v, do), draw(shape, 130, with_grad=True)):
        x.copy_(y)
    bm.copy_(draw_block_mask(N, 131, 0.5, heads=(B, H)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        log(f"case block-sparse graph replay {r}")
        for x, y in zip((q, k, v, do), draw(shape, 132 + r, with_grad=True)):
            x.copy_(y)
        bm.copy_(draw_block_mask(N, 140 + r, 0.5, heads=(B, H), diagonal=r != 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        eo, el = fa_forward_block_sparse(q, k, v, bm, -1, 0)
        eg = fa_backward_block_sparse(q, k, v, eo, do, el, bm, -1, 0)
        torch.cuda.synchronize()
        for a, b in zip(got, (eo, el, *eg)):
            assert torch.equal(a, b), f"replay {r}"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_block_sparse_writes_every_output(d):
    """Outputs preallocated as NaN: every element is written, including the
    rows that see no key (O = 0, lse = -inf, dQ = 0) and the keys no row
    sees (dK = dV = 0)."""
    B, H, Hkv, N = 1, 2, 1, 450
    q, k, v, do = (x.to(DEV) for x in draw((B, H, N, d), 150 + d, with_grad=True, kv_heads=Hkv))
    bm = draw_block_mask(N, 151 + d, 0.4, heads=(B, H), diagonal=False, empty_rows=1).to(DEV)
    bm[:, :, :, 2] = 0  # key block 2 is seen by no row
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full((B, H, N), nan, device=DEV)
    dq, dk, dv = torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(v, nan)
    log(f"case block-sparse poisoned outputs d={d}")
    fa_forward_block_sparse(q, k, v, bm, -1, -1, o=o, lse=lse)
    fa_backward_block_sparse(q, k, v, o, do, lse, bm, -1, -1, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert not torch.isnan(lse).any()
    for x in (o, dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    empty = torch.isneginf(lse)
    assert empty.any()
    assert torch.all(o[empty] == 0) and torch.all(dq[empty] == 0)
    assert torch.all(dk[:, :, 256:384] == 0) and torch.all(dv[:, :, 256:384] == 0)
