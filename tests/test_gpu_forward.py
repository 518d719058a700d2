"""GPU parity of the forward pass (HIP kernels via the C ABI) against the fp64 oracle."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_14_amd import fa_forward, fa_forward_block_sparse, fa_forward_f32
from exact_io_aware_14_amd.inputs import WORKLOADS, draw, to_f64
from parity import check_lse, check_o, check_o_peaked, log, sample_heads, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run_and_compare(shape, causal, seed, scale=None, q_mul=1.0):
    B, H, N, d = shape
    q, k, v = draw(shape, seed)
    if q_mul != 1.0:
        q = (q.float() * q_mul).to(torch.bfloat16)
    # N(0,1) inputs at scale 1/sqrt(d) use the standard gates; others the derived bound
    nominal = scale is None and q_mul == 1.0
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    log(f"case shape={shape} causal={causal} seed={seed} scale={scale} q_mul={q_mul}")
    o, lse = fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    for b in range(B):
        for h in range(H):
            ro, rl = oracle.forward_head(qf[b, h], kf[b, h], vf[b, h], scale, causal)
            if nominal:
                check_o(o[b, h], ro, f"b={b} h={h}")
            else:
                check_o_peaked(o[b, h], ro, np.max(np.abs(vf[b, h])), f"b={b} h={h}")
            check_lse(lse[b, h], rl, f"b={b} h={h}")


SMALL = [
    ((1, 1, 1, 64), False), ((1, 1, 1, 128), True),
    ((1, 1, 17, 64), True), ((1, 2, 64, 128), False),
    ((1, 1, 128, 64), True), ((2, 1, 129, 128), True),
    ((1, 2, 200, 64), False), ((1, 1, 255, 128), False),
    ((1, 1, 256, 128), True), ((2, 3, 333, 64), True),
    ((1, 1, 1000, 128), True), ((1, 1, 1000, 64), False),
    ((1, 8, 384, 128), True), ((2, 4, 512, 64), True),
]


@pytest.mark.parametrize("shape,causal", SMALL, ids=[f"{s}-{'c' if c else 'n'}" for s, c in SMALL])
def test_forward_small(shape, causal):
    _run_and_compare(shape, causal, seed=100 + shape[2])


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_forward_scales(scale, d):
    _run_and_compare((1, 2, 300, d), True, seed=7, scale=scale)
    _run_and_compare((1, 1, 190, d), False, seed=8, scale=scale)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_forward_peaked_rows(d):
    # Q x 8: sharply peaked softmax rows, the running maximum moves often
    _run_and_compare((1, 2, 700, d), True, seed=9, q_mul=8.0)
    _run_and_compare((1, 2, 700, d), False, seed=10, q_mul=8.0)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_forward_max_moves_every_tile(d):
    # scores grow along the keys: every key tile raises every row maximum,
    # by ~30 in units of log2 per tile
    N = 640
    B, H = 1, 1
    q = torch.zeros((B, H, N, d))
    q[..., 0] = 1.0
    k = torch.zeros((B, H, N, d))
    k[..., 0] = torch.arange(N, dtype=torch.float32) * (0.3 * math.sqrt(d))
    g = torch.Generator().manual_seed(5)
    v = torch.randn((B, H, N, d), generator=g)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    for causal in (True, False):
        scale = 1.0 / math.sqrt(d)
        o, lse = fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal)
        torch.cuda.synchronize()
        ro, rl = oracle.forward_head(to_f64(q)[0, 0], to_f64(k)[0, 0], to_f64(v)[0, 0], scale, causal)
        check_o_peaked(o.float().cpu().numpy()[0, 0], ro, np.max(np.abs(to_f64(v))),
                       f"growing causal={causal}")
        check_lse(lse.cpu().numpy()[0, 0], rl, f"growing causal={causal}")


def test_forward_large_offset():
    # a large common offset on every score: exercises the max subtraction
    d = 128
    q, k, v = draw((1, 1, 300, d), 21)
    k = k.float()
    k[..., 1] += 60.0
    q = q.float()
    q[..., 1] = 2.0
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    o, lse = fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=1.0 / math.sqrt(d), causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.forward_head(to_f64(q)[0, 0], to_f64(k)[0, 0], to_f64(v)[0, 0],
                                 1.0 / math.sqrt(d), True)
    check_o_peaked(o.float().cpu().numpy()[0, 0], ro, np.max(np.abs(to_f64(v))), "offset")
    check_lse(lse.cpu().numpy()[0, 0], rl, "offset")


@pytest.mark.parametrize("N", [1, 64, 100, 128, 129, 150, 200, 333, 640, 1000, 8192, 8320])
def test_forward_causal_block_pairs(N):
    """Causal d = 128 launches up to 64 query blocks per head (N <= 8192) give
    each workgroup blocks nqb-1-i and i: odd block counts leave the middle
    block alone, a ragged last block can end on an odd tile count (no tile
    prefetched across the two blocks). Against the oracle (sampled rows at the
    largest lengths), and bitwise against the block-sparse kernel with an
    all-ones mask, which computes every row alike without pairing."""
    B, H, d = 1, 2, 128
    q, k, v = draw((B, H, N, d), 4000 + N)
    log(f"case causal pairs N={N}")
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = fa_forward(qd, kd, vd, causal=True)
    nb = (N + 127) // 128
    ones = torch.ones((nb, nb), dtype=torch.uint8, device=DEV)
    o2, l2 = fa_forward_block_sparse(qd, kd, vd, ones, -1, 0)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    rows = sample_rows(N, seed=N) if N > 2000 else None
    for h in range(H):
        ro, rl = oracle.forward_head(to_f64(q[0, h]), to_f64(k[0, h]), to_f64(v[0, h]),
                                     d ** -0.5, True, rows=rows)
        got_o, got_l = (o[0, h], lse[0, h]) if rows is None else (o[0, h][rows], lse[0, h][rows])
        check_o(got_o, ro, f"N={N} h={h}")
        check_lse(got_l, rl, f"N={N} h={h}")


def test_forward_f32_workload():
    w = WORKLOADS[0]
    q, k, v = draw(w.shape, w.seed, dtype="f32")
    log(f"workload {w.name}")
    o, lse = fa_forward_f32(q.to(DEV), k.to(DEV), v.to(DEV), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    # the kernel rounds the fp32 inputs to bf16; the oracle gets the same rounded values
    qb, kb, vb = (to_f64(x.to(torch.bfloat16)) for x in (q, k, v))
    ro, rl = oracle.forward_head(qb[0, 0], kb[0, 0], vb[0, 0], w.scale, w.causal)
    check_o(o.cpu().numpy()[0, 0], ro, w.name)
    check_lse(lse.cpu().numpy()[0, 0], rl, w.name)
    # information only: distance to the oracle on the unrounded fp32 inputs
    ro32, _ = oracle.forward_head(to_f64(q)[0, 0], to_f64(k)[0, 0], to_f64(v)[0, 0],
                                  w.scale, w.causal)
    log(f"  vs unrounded fp32 inputs: max abs {np.max(np.abs(o.cpu().numpy()[0, 0] - ro32)):.3e}")


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_forward_full_size_workloads(idx):
    """The measured workloads at full size, sampled heads and rows."""
    w = WORKLOADS[idx]
    log(f"workload {w.name}")
    q, k, v = draw(w.shape, w.seed)
    o, lse = fa_forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o = o.cpu()
    lse = lse.cpu()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rows = sample_rows(w.N, seed=w.seed)
    for b, h in sample_heads(w.B, w.H, 4, seed=w.seed):
        ro, rl = oracle.forward_head(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]),
                                     w.scale, w.causal, rows=rows)
        check_o(o[b, h].float().numpy()[rows], ro, f"{w.name} b={b} h={h}")
        check_lse(lse[b, h].numpy()[rows], rl, f"{w.name} b={b} h={h}")


def test_forward_writes_every_output_and_is_deterministic():
    shape = (2, 3, 333, 128)
    q, k, v = (x.to(DEV) for x in draw(shape, 31))
    outs = []
    for _ in range(2):
        o = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full(shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        fa_forward(q, k, v, causal=True, o=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        outs.append((o.clone(), lse.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_forward_leaves_neighbours_untouched():
    shape = (1, 2, 200, 64)
    q, k, v = (x.to(DEV) for x in draw(shape, 32))
    n = int(np.prod(shape))
    canary = 12288.0  # exact in bf16 and fp32
    obuf = torch.full((n + 4096,), canary, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((shape[0] * shape[1] * shape[2] + 1024,), canary, device=DEV)
    o = obuf[:n].view(shape)
    lse = lbuf[: shape[0] * shape[1] * shape[2]].view(shape[:3])
    fa_forward(q, k, v, causal=False, o=o, lse=lse)
    torch.cuda.synchronize()
    assert (obuf[n:].float() == canary).all()
    assert (lbuf[lse.numel():] == canary).all()


def test_forward_empty_is_noop():
    for shape in ((0, 2, 16, 64), (1, 0, 16, 128), (1, 2, 0, 64)):
        q = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        o, lse = fa_forward(q, q, q, causal=True)
        torch.cuda.synchronize()
        assert o.numel() == 0 and lse.numel() == 0
