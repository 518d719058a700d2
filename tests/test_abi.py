"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects invalid arguments with the documented status before any HIP call."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import exact_io_aware_14_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_ALIGN, FA_ERR_ARG, \
    FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_SCRATCH = range(9)


def declared_functions():
    names = []
    for path in HEADERS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \*]*?\b(fa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail(f"{fa.LIB_PATH} not built: run python -m exact_io_aware_14_amd.build")
    return fa.library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"fa_forward", "fa_forward_f32", "fa_backward", "fa_backward_prep",
            "fa_backward_grads", "fa_backward_workspace_size", "fa_strerror",
            "fa_forward_gqa", "fa_backward_gqa", "fa_backward_grads_gqa",
            "fa_forward_window", "fa_backward_window", "fa_backward_grads_window",
            "fa_forward_fp8", "fa_fp8_prepare", "fa_forward_fp8_prepared",
            "fa_forward_fp8_workspace_size", "fa_forward_block_sparse",
            "fa_backward_block_sparse", "fa_backward_grads_block_sparse",
            "fa_backward_noalloc"} <= set(names)
    raw = ctypes.CDLL(fa.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), f"{name} declared in include/ but not exported"


def test_strerror(lib):
    for code in range(9):
        s = fa.fa_strerror(code)
        assert isinstance(s, str) and s
    assert fa.fa_strerror(0) == "success"
    assert fa.fa_strerror(99) == "unknown status"


def test_workspace_size(lib):
    assert fa.fa_backward_workspace_size(4, 16, 4096, 128) == 2 * 4 * 16 * 4096 * 4
    assert fa.fa_backward_workspace_size(4, 8, 4096, 256) == 2 * 4 * 8 * 4096 * 4
    assert fa.fa_backward_workspace_size(1, 1, 1, 64) == 8
    assert fa.fa_backward_workspace_size(0, 1, 1, 64) == 0
    assert fa.fa_backward_workspace_size(1, 1, 1, 96) == 0
    assert fa.fa_backward_workspace_size(1, 1, -5, 64) == 0
    # shapes the calls reject as too large have no workspace size either
    assert fa.fa_backward_workspace_size(1 << 30, 1 << 30, 1 << 30, 128) == 0
    assert fa.fa_backward_workspace_size(1, 1, 1 << 30, 128) == 0
    assert fa.fa_backward_workspace_size(1 << 30, 1 << 30, 1 << 20, 64) == 0


# Fake but aligned device addresses: validation must reject the call before
# it would ever touch them.
P = ctypes.c_void_p(0x10000)
PM = ctypes.c_void_p(0x10008)  # 8-byte aligned only
NULL = ctypes.c_void_p(0)


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, scale=0.125, causal=0, f32=False):
    fn = lib.fa_forward_f32 if f32 else lib.fa_forward
    return fn(q, k, v, o, lse, B, H, N, d, scale, causal, NULL)


def bwd(lib, ws=P, ws_bytes=None, d=64, B=1, H=1, N=16, causal=0, scale=0.125, ptrs=None):
    ptrs = ptrs or [P] * 9
    if ws_bytes is None:
        ws_bytes = 2 * B * H * N * 4 if min(B, H, N) > 0 else 0
    return lib.fa_backward(*ptrs, B, H, N, d, scale, causal, ws, ws_bytes, NULL)


@pytest.mark.parametrize("f32", [False, True])
def test_forward_validation(lib, f32):
    assert fwd(lib, causal=2, f32=f32) == FA_ERR_ARG
    assert fwd(lib, causal=-1, f32=f32) == FA_ERR_ARG
    assert fwd(lib, scale=float("nan"), f32=f32) == FA_ERR_ARG
    assert fwd(lib, scale=float("inf"), f32=f32) == FA_ERR_ARG
    for d in (0, 32, 96, 512, -64):
        assert fwd(lib, d=d, f32=f32) == FA_ERR_HEADDIM
    assert fwd(lib, B=-1, f32=f32) == FA_ERR_SHAPE
    assert fwd(lib, H=-2, f32=f32) == FA_ERR_SHAPE
    assert fwd(lib, N=-3, f32=f32) == FA_ERR_SHAPE
    # the grid would not fit a launch
    assert fwd(lib, B=2**20, H=2**10, N=2**16, f32=f32) == FA_ERR_SHAPE
    # B * H * N past 64 bits: rejected, not wrapped around
    assert fwd(lib, B=2**30, H=2**30, N=2**20, d=64, f32=f32) == FA_ERR_SHAPE
    assert fwd(lib, B=2**31 - 1, H=2**31 - 1, N=2**23, d=64, f32=f32) == FA_ERR_SHAPE
    # one head would not be addressable with 32-bit byte offsets
    assert fwd(lib, N=2**22, d=128, f32=f32) == FA_ERR_SHAPE
    for i in range(5):
        args = [P] * 5
        args[i] = NULL
        assert fwd(lib, *args, f32=f32) == FA_ERR_NULL
        args[i] = PM
        assert fwd(lib, *args, f32=f32) == FA_ERR_ALIGN
    # empty problems are a successful no-op, null pointers allowed
    assert fwd(lib, NULL, NULL, NULL, NULL, NULL, B=0, f32=f32) == FA_OK
    assert fwd(lib, NULL, NULL, NULL, NULL, NULL, H=0, f32=f32) == FA_OK
    assert fwd(lib, NULL, NULL, NULL, NULL, NULL, N=0, f32=f32) == FA_OK


def test_backward_validation(lib):
    assert bwd(lib, causal=3) == FA_ERR_ARG
    assert bwd(lib, scale=float("-inf")) == FA_ERR_ARG
    assert bwd(lib, d=80) == FA_ERR_HEADDIM
    assert bwd(lib, N=-1) == FA_ERR_SHAPE
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = NULL
        assert bwd(lib, ptrs=ptrs) == FA_ERR_NULL
        ptrs[i] = PM
        assert bwd(lib, ptrs=ptrs) == FA_ERR_ALIGN
    assert bwd(lib, ws=NULL) == FA_ERR_WORKSPACE
    assert bwd(lib, ws=PM) == FA_ERR_WORKSPACE
    assert bwd(lib, ws_bytes=2 * 16 * 4 - 1) == FA_ERR_WORKSPACE
    assert bwd(lib, ptrs=[NULL] * 9, ws=NULL, N=0) == FA_OK


def test_backward_stage_validation(lib):
    ws = 2 * 16 * 4
    assert lib.fa_backward_prep(P, P, P, 1, 1, 16, 80, P, ws, NULL) == FA_ERR_HEADDIM
    assert lib.fa_backward_prep(P, P, P, 1, -1, 16, 64, P, ws, NULL) == FA_ERR_SHAPE
    assert lib.fa_backward_prep(NULL, P, P, 1, 1, 16, 64, P, ws, NULL) == FA_ERR_NULL
    assert lib.fa_backward_prep(P, P, NULL, 1, 1, 16, 64, P, ws, NULL) == FA_ERR_NULL
    assert lib.fa_backward_prep(P, PM, P, 1, 1, 16, 64, P, ws, NULL) == FA_ERR_ALIGN
    assert lib.fa_backward_prep(P, P, P, 1, 1, 16, 64, P, ws - 4, NULL) == FA_ERR_WORKSPACE
    assert lib.fa_backward_prep(P, P, P, 1, 1, 16, 64, NULL, ws, NULL) == FA_ERR_WORKSPACE
    assert lib.fa_backward_prep(NULL, NULL, NULL, 1, 1, 0, 64, NULL, 0, NULL) == FA_OK

    def grads(ptrs=None, d=64, N=16, causal=0, scale=0.125, w=P, wb=ws):
        ptrs = ptrs or [P] * 8
        return lib.fa_backward_grads(*ptrs, 1, 1, N, d, scale, causal, w, wb, NULL)
    assert grads(causal=5) == FA_ERR_ARG
    assert grads(scale=float("nan")) == FA_ERR_ARG
    assert grads(d=32) == FA_ERR_HEADDIM
    assert grads(N=-4) == FA_ERR_SHAPE
    for i in range(8):
        ptrs = [P] * 8
        ptrs[i] = NULL
        assert grads(ptrs=ptrs) == FA_ERR_NULL
        ptrs[i] = PM
        assert grads(ptrs=ptrs) == FA_ERR_ALIGN
    assert grads(w=NULL) == FA_ERR_WORKSPACE
    assert grads(wb=ws - 1) == FA_ERR_WORKSPACE
    assert grads(ptrs=[NULL] * 8, N=0, w=NULL, wb=0) == FA_OK


def test_grouped_validation(lib):
    """H_kv must be at least 1 and divide H; the rest is checked as without _gqa."""
    ws = 2 * 6 * 16 * 4

    def fwd_g(H=6, Hkv=2, ptrs=None, N=16, d=64):
        ptrs = ptrs or [P] * 5
        return lib.fa_forward_gqa(*ptrs, 1, H, Hkv, N, d, 0.125, 1, NULL)

    def bwd_g(H=6, Hkv=2, ptrs=None, N=16, d=64, wb=ws):
        ptrs = ptrs or [P] * 9
        return lib.fa_backward_gqa(*ptrs, 1, H, Hkv, N, d, 0.125, 1, P, wb, NULL)

    def grads_g(H=6, Hkv=2, ptrs=None, N=16, d=64, wb=ws):
        ptrs = ptrs or [P] * 8
        return lib.fa_backward_grads_gqa(*ptrs, 1, H, Hkv, N, d, 0.125, 1, P, wb, NULL)

    for call in (fwd_g, bwd_g, grads_g):
        for H, Hkv in ((6, 4), (6, 0), (6, -1), (4, 8), (5, 2)):
            assert call(H=H, Hkv=Hkv) == FA_ERR_SHAPE, (call.__name__, H, Hkv)
        assert call(d=96) == FA_ERR_HEADDIM
        assert call(H=-6) == FA_ERR_SHAPE
        assert call(N=0, ptrs=[NULL] * {fwd_g: 5, bwd_g: 9, grads_g: 8}[call]) == FA_OK
        assert call(H=0, Hkv=0, ptrs=[NULL] * {fwd_g: 5, bwd_g: 9, grads_g: 8}[call]) == FA_OK
    for i in range(5):
        ptrs = [P] * 5
        ptrs[i] = NULL
        assert fwd_g(ptrs=ptrs) == FA_ERR_NULL
    assert bwd_g(wb=ws - 1) == FA_ERR_WORKSPACE
    assert grads_g(wb=ws - 1) == FA_ERR_WORKSPACE


def test_noalloc_validation(lib):
    """fa_backward_noalloc: the checks of fa_backward, then the size of its
    static scratch (B*H*N at most 2^21 rows), all before any HIP call."""
    def call(B=1, H=1, N=16, d=64, causal=0, ptrs=None):
        ptrs = ptrs or [P] * 9
        return lib.fa_backward_noalloc(*ptrs, B, H, N, d, 0.125, causal, NULL)

    assert call(causal=2) == FA_ERR_ARG
    assert call(d=96) == FA_ERR_HEADDIM
    assert call(N=-1) == FA_ERR_SHAPE
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = NULL
        assert call(ptrs=ptrs) == FA_ERR_NULL
        ptrs[i] = PM
        assert call(ptrs=ptrs) == FA_ERR_ALIGN
    assert call(N=0, ptrs=[NULL] * 9) == FA_OK
    assert call(B=1, H=1, N=(2 << 20) + 1) == FA_ERR_SCRATCH
    assert call(B=64, H=32, N=1025) == FA_ERR_SCRATCH
    assert call(B=3, H=5, N=(2 << 20) // 15 + 1, d=128) == FA_ERR_SCRATCH
    assert "scratch" in fa.fa_strerror(FA_ERR_SCRATCH)


def test_window_validation(lib):
    """Window bounds must be >= -1 (-1: none); heads and the rest as for the _gqa calls."""
    ws = 2 * 4 * 16 * 4

    def fwd_w(wl=3, wr=0, H=4, Hkv=2, ptrs=None, N=16, d=64):
        ptrs = ptrs or [P] * 5
        return lib.fa_forward_window(*ptrs, 1, H, Hkv, N, d, 0.125, wl, wr, NULL)

    def bwd_w(wl=3, wr=0, H=4, Hkv=2, ptrs=None, N=16, d=64, wb=ws):
        ptrs = ptrs or [P] * 9
        return lib.fa_backward_window(*ptrs, 1, H, Hkv, N, d, 0.125, wl, wr, P, wb, NULL)

    def grads_w(wl=3, wr=0, H=4, Hkv=2, ptrs=None, N=16, d=64, wb=ws):
        ptrs = ptrs or [P] * 8
        return lib.fa_backward_grads_window(*ptrs, 1, H, Hkv, N, d, 0.125, wl, wr, P, wb, NULL)

    n_ptrs = {fwd_w: 5, bwd_w: 9, grads_w: 8}
    for call in (fwd_w, bwd_w, grads_w):
        for wl, wr in ((-2, 0), (0, -2), (-5, -5)):
            assert call(wl=wl, wr=wr) == FA_ERR_ARG, (call.__name__, wl, wr)
        assert call(H=4, Hkv=3) == FA_ERR_SHAPE
        assert call(d=80) == FA_ERR_HEADDIM
        ptrs = [P] * n_ptrs[call]
        ptrs[0] = NULL
        assert call(ptrs=ptrs) == FA_ERR_NULL
        ptrs[0] = PM
        assert call(ptrs=ptrs) == FA_ERR_ALIGN
        assert call(N=0, ptrs=[NULL] * n_ptrs[call]) == FA_OK
    assert bwd_w(wb=ws - 4) == FA_ERR_WORKSPACE
    assert grads_w(wb=ws - 4) == FA_ERR_WORKSPACE
    # any bound >= -1 is valid, INT_MAX included (a bound of N - 1 or more is
    # no bound): validation goes on to the pointers
    big = 2 ** 31 - 1
    for call in (fwd_w, bwd_w, grads_w):
        for wl, wr in ((big, 0), (-1, big), (big, big), (big - 5, 16)):
            ptrs = [P] * n_ptrs[call]
            ptrs[-1] = PM
            assert call(wl=wl, wr=wr, ptrs=ptrs) == FA_ERR_ALIGN, (call.__name__, wl, wr)


def test_block_sparse_validation(lib):
    """The block-sparse calls check as the _window calls, then the mask: NULL is
    FA_ERR_NULL (after the tensor pointers), a negative head stride FA_ERR_ARG;
    the mask takes any address."""
    ws = 2 * 4 * 16 * 4

    def fwd_s(wl=-1, wr=0, H=4, Hkv=2, ptrs=None, N=16, d=64, m=P, ms=0):
        ptrs = ptrs or [P] * 5
        return lib.fa_forward_block_sparse(*ptrs, 1, H, Hkv, N, d, 0.125, wl, wr, m, ms, NULL)

    def bwd_s(wl=-1, wr=0, H=4, Hkv=2, ptrs=None, N=16, d=64, m=P, ms=0, wb=ws):
        ptrs = ptrs or [P] * 9
        return lib.fa_backward_block_sparse(*ptrs, 1, H, Hkv, N, d, 0.125, wl, wr, m, ms, P, wb,
                                            NULL)

    def grads_s(wl=-1, wr=0, H=4, Hkv=2, ptrs=None, N=16, d=64, m=P, ms=0, wb=ws):
        ptrs = ptrs or [P] * 8
        return lib.fa_backward_grads_block_sparse(*ptrs, 1, H, Hkv, N, d, 0.125, wl, wr, m, ms,
                                                  P, wb, NULL)

    n_ptrs = {fwd_s: 5, bwd_s: 9, grads_s: 8}
    for call in (fwd_s, bwd_s, grads_s):
        assert call(wl=-2) == FA_ERR_ARG
        assert call(m=NULL) == FA_ERR_NULL, call.__name__
        assert call(ms=-1) == FA_ERR_ARG, call.__name__
        assert call(m=NULL, ms=-1) == FA_ERR_NULL
        assert call(m=PM, ms=-1) == FA_ERR_ARG  # a misaligned mask is fine, the stride is not
        assert call(H=4, Hkv=3, m=NULL) == FA_ERR_SHAPE
        assert call(d=80, m=NULL) == FA_ERR_HEADDIM
        ptrs = [P] * n_ptrs[call]
        ptrs[-1] = NULL
        assert call(ptrs=ptrs, m=NULL) == FA_ERR_NULL
        ptrs[-1] = PM
        assert call(ptrs=ptrs, m=NULL) == FA_ERR_ALIGN  # tensor pointers are checked first
        assert call(N=0, ptrs=[NULL] * n_ptrs[call], m=NULL, ms=-1) == FA_OK
    for call in (fwd_s, bwd_s, grads_s):
        assert call(ms=2 ** 62) == FA_ERR_ARG  # (B*H - 1) * stride overflows 64 bits
    assert bwd_s(wb=ws - 4, ms=-1) == FA_ERR_ARG
    assert bwd_s(wb=ws - 4, ms=7) == FA_ERR_WORKSPACE
    assert grads_s(wb=ws - 4, ms=7) == FA_ERR_WORKSPACE


def test_fp8_workspace_size(lib):
    """Regions q8, qs, k8, ks, v8, vs, each rounded up to 256 bytes (T = ceil(N/64))."""
    # B=1, H=2, H_kv=1, N=100, d=64: 12800 + 1024 + 8192 + 256 + 8192 + 512
    assert fa.fa_forward_fp8_workspace_size(1, 2, 1, 100, 64) == 30976
    # B=4, H=16, N=4096, d=128: 32 MiB of each code region, 1 MiB of row factors,
    # 4*16*64 tile scales, 4*16*64 blocks of 256 B of block scales
    T = 64
    want = 2 ** 25 + 4 * 16 * 4096 * 4 + 2 ** 25 + 4 * 16 * T * 4 + 2 ** 25 + 4 * 16 * T * 256
    assert fa.fa_forward_fp8_workspace_size(4, 16, 16, 4096, 128) == want
    assert fa.fa_forward_fp8_workspace_size(0, 2, 1, 100, 64) == 0
    assert fa.fa_forward_fp8_workspace_size(1, 2, 3, 100, 64) == 0
    assert fa.fa_forward_fp8_workspace_size(1, 2, 1, 100, 96) == 0
    assert fa.fa_forward_fp8_workspace_size(1, 2, 1, 100, 256) == 0  # FP8: d = 64 and 128 only


def test_fp8_validation(lib):
    """Signs must be +1/-1 (host array) or NULL; workspace of the documented size;
    the rest as for the _gqa calls."""
    ws = fa.fa_forward_fp8_workspace_size(1, 4, 2, 100, 64)
    good = (ctypes.c_int8 * 64)(*([1, -1] * 32))
    bad = (ctypes.c_int8 * 64)(*([1] * 63 + [0]))
    gp, bp = ctypes.cast(good, ctypes.c_void_p), ctypes.cast(bad, ctypes.c_void_p)

    def fwd(signs=gp, H=4, Hkv=2, N=100, d=64, scale=0.125, causal=1, ptrs=None, w=P, wb=ws):
        ptrs = ptrs or [P] * 5
        return lib.fa_forward_fp8(ptrs[0], ptrs[1], ptrs[2], signs, ptrs[3], ptrs[4], 1, H, Hkv,
                                  N, d, scale, causal, w, wb, NULL)

    def prep(signs=gp, H=4, Hkv=2, N=100, d=64, ptrs=None, w=P, wb=ws):
        ptrs = ptrs or [P] * 3
        return lib.fa_fp8_prepare(*ptrs, signs, 1, H, Hkv, N, d, w, wb, NULL)

    def attn(H=4, Hkv=2, N=100, d=64, scale=0.125, causal=1, ptrs=None, w=P, wb=ws):
        ptrs = ptrs or [P] * 2
        return lib.fa_forward_fp8_prepared(w, wb, ptrs[0], ptrs[1], 1, H, Hkv, N, d, scale,
                                           causal, NULL)

    assert fwd(signs=bp) == FA_ERR_ARG
    assert prep(signs=bp) == FA_ERR_ARG
    for call in (fwd, attn):
        assert call(causal=2) == FA_ERR_ARG
        assert call(scale=float("nan")) == FA_ERR_ARG
    for call, n in ((fwd, 5), (prep, 3), (attn, 2)):
        assert call(H=4, Hkv=3) == FA_ERR_SHAPE
        assert call(d=80) == FA_ERR_HEADDIM
        assert call(d=256) == FA_ERR_HEADDIM
        assert call(w=NULL) == FA_ERR_WORKSPACE
        assert call(wb=ws - 1) == FA_ERR_WORKSPACE
        assert call(w=PM) == FA_ERR_WORKSPACE
        for i in range(n):
            ptrs = [P] * n
            ptrs[i] = NULL
            assert call(ptrs=ptrs) == FA_ERR_NULL, (call.__name__, i)
            ptrs[i] = PM
            assert call(ptrs=ptrs) == FA_ERR_ALIGN, (call.__name__, i)
        assert call(N=0, ptrs=[NULL] * n, w=NULL, wb=0) == FA_OK


def test_python_binding_without_gpu_raises_cleanly(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_forward(q, q, q)  # CPU tensors are refused before the library is called
    k = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_forward_gqa(torch.zeros((1, 2, 4, 64), dtype=torch.bfloat16), k, k)
    with pytest.raises(ValueError):
        fa.fa_forward_block_sparse(q, q, q, torch.ones((1, 1), dtype=torch.uint8))
