"""GPU parity of head dimension 256 (forward, backward, grouped K/V heads,
local windows, fp32 forward) through the C ABI, against the fp64 oracle,
with the same gates as the other head dimensions."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_14_amd import (fa_backward, fa_backward_grads, fa_backward_prep,
                                   fa_backward_workspace_size,
                                   fa_backward_window, fa_forward, fa_forward_f32,
                                   fa_forward_window)
from exact_io_aware_14_amd.inputs import D256_WORKLOADS, draw, to_f64
from parity import check_grad, check_lse, check_o, dq_allowance, dq_allowances, log, sample_heads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D = 256

# (B, H, H_kv, N, window_left, window_right): causal (-1, 0), none (-1, -1),
# local windows, grouped and multi-query K/V heads, ragged N
CASES = [
    (1, 2, 2, 200, -1, 0), (1, 2, 2, 333, -1, -1), (2, 4, 2, 257, -1, 0), (1, 2, 1, 64, -1, -1),
    (1, 1, 1, 1, -1, 0), (1, 2, 2, 1000, -1, 0), (1, 2, 2, 500, 100, 0), (1, 3, 1, 300, 33, 17),
    (1, 2, 2, 129, -1, 40),
]


def _ids(cases):
    return [f"B{b}H{h}kv{hk}N{n}w{l}_{r}" for b, h, hk, n, l, r in cases]


@pytest.mark.parametrize("case", CASES, ids=_ids(CASES))
def test_d256_forward(case):
    B, H, Hkv, N, wl, wr = case
    scale = 1.0 / math.sqrt(D)
    log(f"case d256 forward {case}")
    q, k, v = draw((B, H, N, D), 1100 + N, kv_heads=Hkv)
    o, lse = fa_forward_window(q.to(DEV), k.to(DEV), v.to(DEV), wl, wr, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for h in range(H):
            g = oracle.kv_head(h, H, Hkv)
            ro, rl = oracle.forward_head(to_f64(q[b, h]), to_f64(k[b, g]), to_f64(v[b, g]),
                                         scale, (wl, wr))
            check_o(o[b, h], ro, f"{case} b={b} h={h}")
            check_lse(lse[b, h], rl, f"{case} b={b} h={h}")


@pytest.mark.parametrize("case", CASES, ids=_ids(CASES))
def test_d256_backward(case):
    B, H, Hkv, N, wl, wr = case
    scale = 1.0 / math.sqrt(D)
    log(f"case d256 backward {case}")
    q, k, v, do = draw((B, H, N, D), 1200 + N, with_grad=True, kv_heads=Hkv)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_forward_window(qd, kd, vd, wl, wr, scale=scale)
    dq, dk, dv = fa_backward_window(qd, kd, vd, o, dod, lse, wl, wr, scale=scale)
    torch.cuda.synchronize()
    args = (to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, (wl, wr))
    rq, rk, rv = oracle.backward(*args)
    aq = dq_allowances(*args)
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    for b in range(B):
        for h in range(H):
            check_grad(dq[b, h], rq[b, h], f"{case} b={b} h={h} dQ", allow=aq[b, h])
        for g in range(Hkv):
            check_grad(dk[b, g], rk[b, g], f"{case} b={b} kv={g} dK")
            check_grad(dv[b, g], rv[b, g], f"{case} b={b} kv={g} dV")


def test_d256_plain_calls_and_stages():
    """fa_forward / fa_backward (multi-head, causal flag) at d = 256 equal the
    window calls with (-1, 0) / (-1, -1) bitwise, and prep + grads equal
    fa_backward bitwise."""
    shape = (1, 2, 300, D)
    q, k, v, do = (x.to(DEV) for x in draw(shape, 71, with_grad=True))
    for causal, win in ((True, (-1, 0)), (False, (-1, -1))):
        o1, l1 = fa_forward(q, k, v, causal=causal)
        o2, l2 = fa_forward_window(q, k, v, *win)
        g1 = fa_backward(q, k, v, o1, do, l1, causal=causal)
        g2 = fa_backward_window(q, k, v, o1, do, l1, *win)
        ws = fa_backward_prep(o1, do, l1)
        g3 = fa_backward_grads(q, k, v, do, l1, ws, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for a, b, c in zip(g1, g2, g3):
            assert torch.equal(a, b) and torch.equal(a, c)


def test_d256_forward_f32():
    """fp32 in/out at d = 256: inputs rounded to bf16 on load, fp32 output."""
    B, H, N = 1, 2, 130
    q, k, v = draw((B, H, N, D), 72, dtype="f32")
    o, lse = fa_forward_f32(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    for h in range(H):
        args = [to_f64(x[0, h].to(torch.bfloat16)) for x in (q, k, v)]
        ro, rl = oracle.forward_head(*args, D ** -0.5, True)
        check_o(o[0, h], ro, f"f32 h={h}")
        check_lse(lse[0, h].cpu().numpy(), rl, f"f32 h={h}")


def test_d256_full_size_workload():
    """B=4, H=8, N=4096, d=256, causal: sampled heads of O, one head's gradients."""
    w = D256_WORKLOADS[0]
    log(f"workload {w.name}")
    q, k, v, do = draw(w.shape, w.seed, with_grad=True)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_forward(qd, kd, vd, scale=w.scale, causal=True)
    dq, dk, dv = fa_backward(qd, kd, vd, o, dod, lse, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for x in (o, dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    o = o.float().cpu().numpy()
    for b, h in sample_heads(w.B, w.H, 2, seed=w.seed):
        ro, rl = oracle.forward_head(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), w.scale,
                                     True)
        check_o(o[b, h], ro, f"{w.name} b={b} h={h}")
        check_lse(lse[b, h].cpu().numpy(), rl, f"{w.name} b={b} h={h}")
    b, h = 3, 7
    args = (to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), to_f64(do[b, h]), w.scale, True)
    rq, rk, rv = oracle.backward_head(*args)
    aq = dq_allowance(*args)
    for name, got, ref, al in (("dQ", dq, rq, aq), ("dK", dk, rk, None), ("dV", dv, rv, None)):
        check_grad(got[b, h].float().cpu().numpy(), ref, f"{w.name} b={b} h={h} {name}",
                   allow=al)


def test_d256_writes_every_output_and_is_deterministic():
    """NaN-poisoned outputs and workspace: every element written, two calls
    bitwise equal, forward and backward."""
    shape = (1, 3, 333, D)
    q, k, v, do = (x.to(DEV) for x in draw(shape, 73, with_grad=True))
    results = []
    for _ in range(2):
        o = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full(shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        fa_forward(q, k, v, causal=True, o=o, lse=lse)
        grads = [torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
                 for _ in range(3)]
        ws = torch.full((fa_backward_workspace_size(*shape) // 4,), float("nan"), device=DEV)
        fa_backward(q, k, v, o, do, lse, causal=True, dq=grads[0], dk=grads[1], dv=grads[2],
                    workspace=ws)
        torch.cuda.synchronize()
        for x in [o, lse] + grads:
            assert torch.isfinite(x.float()).all()
        results.append([x.clone() for x in [o, lse] + grads])
    for a, b in zip(results[0], results[1]):
        assert torch.equal(a, b)


def test_d256_leaves_neighbours_untouched():
    shape = (1, 2, 200, D)
    q, k, v, do = (x.to(DEV) for x in draw(shape, 74, with_grad=True))
    n = int(np.prod(shape))
    canary = 12288.0
    bufs = [torch.full((n + 4096,), canary, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    lbuf = torch.full((shape[0] * shape[1] * shape[2] + 1024,), canary, device=DEV)
    o, dq, dk, dv = (b[:n].view(shape) for b in bufs)
    lse = lbuf[: shape[0] * shape[1] * shape[2]].view(shape[:3])
    fa_forward(q, k, v, causal=False, o=o, lse=lse)
    fa_backward(q, k, v, o, do, lse, causal=False, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for b in bufs:
        assert (b[n:].float() == canary).all()
    assert (lbuf[lse.numel():] == canary).all()
