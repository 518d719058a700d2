"""fa_backward_noalloc, the backward whose row terms live in the library's
static scratch (for callers that cannot allocate), through the C ABI against
fa_backward, the entry point with a caller workspace: both run the same
kernels on the same inputs, so the results must agree bitwise. Two calls in a
row, the second on a smaller input (the scratch keeps the first call's
contents), then the largest problem the scratch holds; and the call captured
in a HIP graph (the use it is for), replayed on new inputs."""

from __future__ import annotations

import pytest
import torch

from exact_io_aware_14_amd import FAError, fa_backward, fa_backward_noalloc, fa_forward
from exact_io_aware_14_amd.inputs import draw
from parity import log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FA_ERR_SCRATCH = 8
MAX_ROWS = 2 << 20  # B * H * N the static scratch holds


def _compare(shape, causal, seed):
    q, k, v, do = (x.to(DEV) for x in draw(shape, seed, with_grad=True))
    o, lse = fa_forward(q, k, v, causal=causal)
    ref = fa_backward(q, k, v, o, do, lse, causal=causal)
    outs = [torch.full_like(q, float("nan")) for _ in range(3)]
    got = fa_backward_noalloc(q, k, v, o, do, lse, causal=causal, dq=outs[0], dk=outs[1],
                              dv=outs[2])
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, b), f"{shape} causal={causal} {name}"


def test_noalloc_matches_backward_on_two_calls():
    for shape, causal, seed in (((2, 4, 1000, 128), True, 91), ((1, 2, 300, 64), False, 92)):
        log(f"case noalloc {shape} causal={causal}")
        _compare(shape, causal, seed)


def test_noalloc_largest_problem_and_limit():
    shape = (64, 32, 1024, 64)
    assert shape[0] * shape[1] * shape[2] == MAX_ROWS
    log(f"case noalloc {shape} causal=True (the scratch's largest problem)")
    _compare(shape, True, 93)
    log("case noalloc d=256 after it")
    _compare((1, 2, 200, 256), True, 94)
    # one row more than the scratch holds: rejected before any launch
    q = torch.zeros((1, 1, MAX_ROWS + 1, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((1, 1, MAX_ROWS + 1), dtype=torch.float32, device=DEV)
    with pytest.raises(FAError) as err:
        fa_backward_noalloc(q, q, q, q, q, lse, dq=q, dk=q, dv=q)
    assert err.value.status == FA_ERR_SCRATCH


def test_noalloc_graph_replays_match_backward():
    """Forward + fa_backward_noalloc captured once, replayed three times on new
    input contents with eager work and synchronisations between replays; each
    replay bitwise equal to eager fa_forward + fa_backward."""
    shape = (2, 4, 333, 128)
    B, H, N, d = shape
    q, k, v, do = (torch.empty(shape, dtype=torch.bfloat16, device=DEV) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)

    def step():
        fa_forward(q, k, v, causal=True, o=o, lse=lse)
        fa_backward_noalloc(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv)

    for x, y in zip((q, k, v, do), draw(shape, 95, with_grad=True)):
        x.copy_(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for r in range(3):
        log(f"case noalloc graph replay {r}")
        for x, y in zip((q, k, v, do), draw(shape, 96 + r, with_grad=True)):
            x.copy_(y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        eo, el = fa_forward(q, k, v, causal=True)
        eg = fa_backward(q, k, v, eo, do, el, causal=True)
        torch.cuda.synchronize()
        for a, b in zip(got, (eo, el, *eg)):
            assert torch.equal(a, b), f"replay {r}"
