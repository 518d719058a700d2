"""Whole-output identities of the GPU kernels at full workload sizes (no oracle).

The parity tests compare sampled rows of the full-size workloads with the
fp64 oracle. Here every row of a full-size output is checked against an
identity the mathematics fixes, computed from other launches of the
kernels: the decomposition of the softmax over a split key set (unite.ai
page, softmax decomposition and merge). Attention over keys [0, N/2) and
over keys [N/2, N) -- two block-sparse launches whose masks keep the lower
and the upper half of the key blocks -- merged through their logsumexps
must give the attention over all keys of one plain launch:

    lse = log(exp(lse_1) + exp(lse_2)),
    O   = exp(lse_1 - lse) O_1 + exp(lse_2 - lse) O_2

(a part with no visible key has lse = -inf and weight 0). A wrong or
missing tile in any head or row of either path shows up in that row.

The merge runs in fp32 on the GPU from the bf16 partial outputs, so the
merged O carries one more bf16 rounding than the direct one; the gates
are those of O and lse against the oracle.
"""
import pytest
import torch

from exact_io_aware_14_amd import fa_forward, fa_forward_block_sparse, fa_forward_gqa
from exact_io_aware_14_amd.inputs import MASK_BLOCK, by_name, draw
from parity import LSE_MAX_ABS, O_MAX_ABS, O_REL_L2, log

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _merge(o1, l1, o2, l2):
    lse = torch.logaddexp(l1, l2)
    w1 = torch.where(torch.isfinite(l1), torch.exp(l1 - lse), torch.zeros_like(l1))
    w2 = torch.where(torch.isfinite(l2), torch.exp(l2 - lse), torch.zeros_like(l2))
    return w1[..., None] * o1.float() + w2[..., None] * o2.float(), lse


def _split_masks(N):
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    cols = torch.arange(nb, device=DEV)[None, :].expand(nb, nb)
    lower = (cols < nb // 2).to(torch.uint8).contiguous()
    return lower, (1 - lower).contiguous()


@pytest.mark.parametrize("name,causal", [
    ("fwd_causal_b1h16n32768d128", True),   # the long-sequence workload
    ("fwd_b8h16n2048d64", False),            # d = 64, no mask
    ("fwdbwd_causal_b4h8n4096d256", True),   # d = 256 (32-key tiles)
])
def test_split_keys_merge_to_the_full_output(name, causal):
    w = by_name(name)
    log(f"case merge identity {name} causal={causal}")
    q, k, v = (x.to(DEV) for x in draw(w.shape, w.seed)[:3])
    wl, wr = (-1, 0) if causal else (-1, -1)
    if w.d == 256:
        o, lse = fa_forward_gqa(q, k, v, scale=w.scale, causal=causal)
    else:
        o, lse = fa_forward(q, k, v, scale=w.scale, causal=causal)
    lower, upper = _split_masks(w.N)
    o1, l1 = fa_forward_block_sparse(q, k, v, lower, wl, wr, scale=w.scale)
    o2, l2 = fa_forward_block_sparse(q, k, v, upper, wl, wr, scale=w.scale)
    om, lm = _merge(o1, l1, o2, l2)
    torch.cuda.synchronize()
    of = o.float()
    diff = (om - of).abs()
    max_abs = float(diff.max())
    rel = float(torch.linalg.vector_norm(om - of) / torch.linalg.vector_norm(of))
    lse_abs = float((lm - lse).abs().max())
    # the worst row, relative to its own norm
    row_rel = float(((om - of).norm(dim=-1) / of.norm(dim=-1).clamp_min(1e-6)).max())
    log(f"  max_abs={max_abs:.3e} rel_l2={rel:.3e} lse_max_abs={lse_abs:.3e} worst_row_rel={row_rel:.3e}")
    assert torch.isfinite(om).all() and torch.isfinite(lm).all()
    assert max_abs <= O_MAX_ABS and rel <= O_REL_L2, (name, max_abs, rel)
    assert lse_abs <= LSE_MAX_ABS, (name, lse_abs)
    assert row_rel <= 2e-2, (name, row_rel)
