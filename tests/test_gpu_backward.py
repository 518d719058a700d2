"""GPU parity of the backward pass (HIP kernels via the C ABI) against the fp64 oracle."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_14_amd import (fa_backward, fa_backward_grads, fa_backward_prep,
                                   fa_backward_workspace_size, fa_forward)
from exact_io_aware_14_amd.inputs import WORKLOADS, draw, to_f64
from parity import check_grad, check_o, dq_allowance, log, sample_heads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fwd_bwd(q, k, v, do, scale, causal):
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_forward(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = fa_backward(qd, kd, vd, o, dod, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _compare_heads(q, k, v, do, scale, causal, heads, outs, what):
    _, _, dq, dk, dv = outs
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    for b, h in heads:
        args = (to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), to_f64(do[b, h]), scale, causal)
        rq, rk, rv = oracle.backward_head(*args)
        check_grad(dq[b, h], rq, f"{what} b={b} h={h} dQ", allow=dq_allowance(*args))
        check_grad(dk[b, h], rk, f"{what} b={b} h={h} dK")
        check_grad(dv[b, h], rv, f"{what} b={b} h={h} dV")


SMALL = [
    ((1, 1, 1, 64), True), ((1, 1, 1, 128), False),
    ((1, 1, 17, 128), True), ((1, 2, 64, 64), False),
    ((1, 1, 129, 128), True), ((2, 2, 200, 64), True),
    ((1, 1, 333, 128), False), ((1, 1, 333, 128), True),
    ((1, 2, 1000, 128), True), ((1, 2, 1000, 64), False),
    ((1, 8, 256, 128), True), ((2, 4, 384, 64), True),
]


@pytest.mark.parametrize("shape,causal", SMALL, ids=[f"{s}-{'c' if c else 'n'}" for s, c in SMALL])
def test_backward_small(shape, causal):
    B, H, N, d = shape
    q, k, v, do = draw(shape, 200 + N, with_grad=True)
    scale = 1.0 / math.sqrt(d)
    log(f"case shape={shape} causal={causal}")
    outs = _fwd_bwd(q, k, v, do, scale, causal)
    heads = [(b, h) for b in range(B) for h in range(H)]
    _compare_heads(q, k, v, do, scale, causal, heads, outs, str(shape))


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.35])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_scales(scale, d):
    shape = (1, 2, 300, d)
    q, k, v, do = draw(shape, 41, with_grad=True)
    for causal in (True, False):
        log(f"case shape={shape} causal={causal} scale={scale}")
        outs = _fwd_bwd(q, k, v, do, scale, causal)
        _compare_heads(q, k, v, do, scale, causal, [(0, 0), (0, 1)], outs, f"scale={scale}")


def test_backward_full_size_workload():
    """The forward+backward workload at full size: two whole heads compared."""
    w = WORKLOADS[4]
    log(f"workload {w.name}")
    q, k, v, do = draw(w.shape, w.seed, with_grad=True)
    outs = _fwd_bwd(q, k, v, do, w.scale, w.causal)
    for x in outs[2:]:
        assert torch.isfinite(x.float()).all()
    heads = sample_heads(w.B, w.H, 2, seed=w.seed)
    o = outs[0].float().cpu().numpy()
    for b, h in heads:
        ro, _ = oracle.forward_head(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]),
                                    w.scale, w.causal)
        check_o(o[b, h], ro, f"{w.name} b={b} h={h}")
    _compare_heads(q, k, v, do, w.scale, w.causal, heads, outs, w.name)


LARGE = [((1, 16, 16384, 128), True, 11), ((2, 16, 4096, 64), False, 13), ((1, 8, 8192, 256), True, 5)]


@pytest.mark.parametrize("shape,causal,h", LARGE, ids=[f"{s}-{'c' if c else 'n'}" for s, c, _ in LARGE])
def test_backward_large_shapes(shape, causal, h):
    """Long sequences and every head dimension at full launch size: one whole
    head's gradients and the first and last 256 rows of its output against
    the oracle (which holds that head's full N x N matrices in fp64: about
    10 GB at N = 16384)."""
    scale = 1.0 / math.sqrt(shape[3])
    q, k, v, do = draw(shape, 47 + shape[2] + shape[3], with_grad=True)
    log(f"case large {shape} causal={causal} head {h}")
    outs = _fwd_bwd(q, k, v, do, scale, causal)
    for x in outs[2:]:
        assert torch.isfinite(x.float()).all()
    b = shape[0] - 1
    rows = np.concatenate([np.arange(256), np.arange(shape[2] - 256, shape[2])])
    ro, _ = oracle.forward_head(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), scale, causal,
                                rows=rows)
    check_o(outs[0][b, h].float().cpu().numpy()[rows], ro, f"{shape} b={b} h={h}")
    _compare_heads(q, k, v, do, scale, causal, [(b, h)], outs, str(shape))


def test_backward_writes_every_output_and_is_deterministic():
    shape = (2, 2, 333, 128)
    q, k, v, do = (x.to(DEV) for x in draw(shape, 43, with_grad=True))
    o, lse = fa_forward(q, k, v, causal=True)
    results = []
    for _ in range(2):
        grads = [torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
                 for _ in range(3)]
        ws = torch.full((fa_backward_workspace_size(*shape) // 4,), float("nan"), device=DEV)
        fa_backward(q, k, v, o, do, lse, causal=True, dq=grads[0], dk=grads[1], dv=grads[2],
                    workspace=ws)
        torch.cuda.synchronize()
        for g in grads:
            assert torch.isfinite(g.float()).all()
        results.append([g.clone() for g in grads])
    for a, b in zip(results[0], results[1]):
        assert torch.equal(a, b)


def test_backward_stages_match_backward():
    """fa_backward_prep + fa_backward_grads give bitwise the result of fa_backward."""
    for shape, causal in (((2, 2, 333, 128), True), ((1, 3, 200, 64), False)):
        q, k, v, do = (x.to(DEV) for x in draw(shape, 44, with_grad=True))
        o, lse = fa_forward(q, k, v, causal=causal)
        ref = fa_backward(q, k, v, o, do, lse, causal=causal)
        ws = fa_backward_prep(o, do, lse)
        # the row terms are D_i = sum_k dO_ik O_ik, then lse_i * log2(e)
        rows = shape[0] * shape[1] * shape[2]
        terms = ws[: 2 * rows * 4].view(torch.float32)
        expect = (do.float() * o.float()).sum(-1).reshape(-1)
        assert torch.allclose(terms[:rows], expect, rtol=1e-5, atol=1e-5)
        assert torch.allclose(terms[rows:], lse.reshape(-1) * 1.4426950408889634, rtol=1e-6)
        got = fa_backward_grads(q, k, v, do, lse, ws, causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)


def test_backward_empty_is_noop():
    for shape in ((0, 1, 8, 64), (1, 1, 0, 128)):
        z = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(shape[:3], dtype=torch.float32, device=DEV)
        dq, dk, dv = fa_backward(z, z, z, z, z, lse, causal=True)
        torch.cuda.synchronize()
        assert dq.numel() == 0


@pytest.mark.parametrize("d", [64, 128, 256])
def test_many_short_heads(d):
    """B*H = 4096 heads of 17 rows (every K/V head count a multiple of 8, so the
    launches hand heads to XCDs whole): sampled heads against the oracle."""
    shape = (64, 64, 17, d)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = draw(shape, 48 + d, with_grad=True)
    for causal in (True, False):
        log(f"case many short heads {shape} causal={causal}")
        outs = _fwd_bwd(q, k, v, do, scale, causal)
        heads = sample_heads(shape[0], shape[1], 6, seed=d)
        o = outs[0].float().cpu().numpy()
        for b, h in heads:
            ro, _ = oracle.forward_head(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), scale,
                                        causal)
            check_o(o[b, h], ro, f"{shape} b={b} h={h}")
        _compare_heads(q, k, v, do, scale, causal, heads, outs, f"many heads d={d}")
