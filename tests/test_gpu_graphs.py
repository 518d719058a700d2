"""The C ABI under HIP graph capture: the calls allocate nothing, set no
memory and never synchronise, so a forward + backward (and the FP8 forward)
captured once replays like eager calls. Each replay runs on new input
contents, with eager work and synchronisations between replays, and every
replay is compared with eager calls on the same inputs, bitwise."""

from __future__ import annotations

import pytest
import torch

from exact_io_aware_14_amd import (fa_backward, fa_backward_workspace_size, fa_forward,
                                   fa_forward_fp8, fa_forward_fp8_workspace_size,
                                   fa_forward_window)
from exact_io_aware_14_amd.inputs import draw, draw_signs
from parity import log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_forward_backward_graph_replays_match_eager():
    shape = (2, 4, 333, 128)
    B, H, N, d = shape
    q, k, v, do = (torch.empty(shape, dtype=torch.bfloat16, device=DEV) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa_backward_workspace_size(*shape), dtype=torch.uint8, device=DEV)
    ow = torch.empty_like(q)
    lsew = torch.empty_like(lse)

    def step():
        fa_forward(q, k, v, causal=True, o=o, lse=lse)
        fa_backward(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
        fa_forward_window(q, k, v, 50, 7, o=ow, lse=lsew)

    for x, y in zip((q, k, v, do), draw(shape, 81, with_grad=True)):
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
        log(f"case graph replay {r}")
        for x, y in zip((q, k, v, do), draw(shape, 90 + r, with_grad=True)):
            x.copy_(y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv, ow, lsew)]
        eo, el = fa_forward(q, k, v, causal=True)
        eg = fa_backward(q, k, v, eo, do, el, causal=True)
        ew = fa_forward_window(q, k, v, 50, 7)
        torch.cuda.synchronize()
        for a, b in zip(got, (eo, el, *eg, *ew)):
            assert torch.equal(a, b), f"replay {r}"


def test_fp8_forward_graph_replays_match_eager():
    shape = (1, 4, 300, 128)
    B, H, N, d = shape
    q, k, v = (torch.empty(shape, dtype=torch.bfloat16, device=DEV) for _ in range(3))
    signs = draw_signs(d, 82)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=DEV)
    ws = torch.empty(fa_forward_fp8_workspace_size(B, H, H, N, d), dtype=torch.uint8, device=DEV)

    def step():
        fa_forward_fp8(q, k, v, signs, causal=True, o=o, lse=lse, workspace=ws)

    for x, y in zip((q, k, v), draw(shape, 83)):
        x.copy_(y)
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
        log(f"case fp8 graph replay {r}")
        for x, y in zip((q, k, v), draw(shape, 95 + r)):
            x.copy_(y)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone())
        eo, el = fa_forward_fp8(q, k, v, signs, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(got[0], eo) and torch.equal(got[1], el), f"replay {r}"
