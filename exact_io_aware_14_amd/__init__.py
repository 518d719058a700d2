"""Exact tiled attention on MI355X (gfx950): Python binding of libfa.so.

The functions here carry the names of the C ABI in include/fa.h and only
marshal arguments: they check torch tensors (device, dtype, contiguity,
shape), allocate missing outputs with torch, and pass raw device pointers and
the HIP stream (the one given, else torch's current stream) to the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback. If libfa.so has not been built, every call raises.
"""

from __future__ import annotations

import ctypes
import os

__all__ = ["FAError", "fa_forward", "fa_forward_gqa", "fa_forward_window", "fa_forward_f32",
           "fa_backward", "fa_backward_noalloc", "fa_backward_gqa", "fa_backward_window", "fa_backward_prep",
           "fa_backward_grads", "fa_backward_grads_gqa", "fa_backward_grads_window",
           "fa_forward_block_sparse", "fa_backward_block_sparse",
           "fa_backward_grads_block_sparse", "MASK_BLOCK",
           "fa_backward_workspace_size", "fa_forward_fp8", "fa_fp8_prepare",
           "fa_forward_fp8_prepared", "fa_forward_fp8_workspace_size", "fa_strerror", "library",
           "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

MASK_BLOCK = 128  # query rows and keys per block of a block-sparse mask

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status}: {fa_strerror(status)}")
        self.status = status


def library():
    """The loaded libfa.so (ctypes). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_14_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        ll = ctypes.c_longlong
        lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_forward.restype = i
        lib.fa_forward_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_forward_f32.restype = i
        for name, argtypes in (
                ("fa_forward_gqa", [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]),
                ("fa_backward_gqa", [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                                     vp, sz, vp]),
                ("fa_backward_grads_gqa", [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                                           vp, sz, vp]),
                ("fa_forward_window", [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]),
                ("fa_backward_window", [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                                        i, vp, sz, vp]),
                ("fa_backward_grads_window", [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f,
                                              i, i, vp, sz, vp]),
                ("fa_forward_fp8", [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]),
                ("fa_fp8_prepare", [vp, vp, vp, vp, i, i, i, i, i, vp, sz, vp]),
                ("fa_forward_fp8_prepared", [vp, sz, vp, vp, i, i, i, i, i, f, i, vp]),
                ("fa_forward_block_sparse", [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, ll,
                                             vp]),
                ("fa_backward_block_sparse", [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i,
                                              f, i, i, vp, ll, vp, sz, vp]),
                ("fa_backward_grads_block_sparse", [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i,
                                                    i, f, i, i, vp, ll, vp, sz, vp])):
            if hasattr(lib, name):  # an older build without them fails when they are called
                getattr(lib, name).argtypes = argtypes
                getattr(lib, name).restype = i
        if hasattr(lib, "fa_forward_fp8_workspace_size"):
            lib.fa_forward_fp8_workspace_size.argtypes = [i, i, i, i, i]
            lib.fa_forward_fp8_workspace_size.restype = sz
        lib.fa_backward_workspace_size.argtypes = [i, i, i, i]
        lib.fa_backward_workspace_size.restype = sz
        lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i,
                                    vp, sz, vp]
        lib.fa_backward.restype = i
        if hasattr(lib, "fa_backward_noalloc"):
            lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f,
                                                i, vp]
            lib.fa_backward_noalloc.restype = i
        lib.fa_backward_prep.argtypes = [vp, vp, vp, i, i, i, i, vp, sz, vp]
        lib.fa_backward_prep.restype = i
        lib.fa_backward_grads.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i,
                                          vp, sz, vp]
        lib.fa_backward_grads.restype = i
        lib.fa_strerror.argtypes = [i]
        lib.fa_strerror.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def fa_strerror(status: int) -> str:
    return library().fa_strerror(int(status)).decode()


def fa_backward_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(library().fa_backward_workspace_size(B, H, N, d))


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream, *tensors):
    """The HIP stream handle of a call: `stream` (a torch stream or a raw
    handle), else torch's current stream. On any other stream than the
    current one, the tensors the call reads or writes are recorded on it, so
    that torch's caching allocator hands their memory to no other work before
    the call's kernels are done: the binding's own temporaries (outputs and
    workspaces it allocated) are freed as soon as the caller drops them,
    possibly while the kernels still run."""
    torch = _torch()
    current = torch.cuda.current_stream()
    if stream is None:
        return ctypes.c_void_p(current.cuda_stream)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if handle != current.cuda_stream:
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(handle)
        for t in tensors:
            if t is not None:
                t.record_stream(s)
    return ctypes.c_void_p(handle)


def _check(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on {device} (a HIP device)")


def _kv_heads(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d] and [B, H_kv, N, d]")
    return k.shape[1]


def _forward(fn_name, q, k, v, scale, causal, o, lse, stream, dtype, gqa=False, window=None):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(q, k) if gqa else H
    dev = q.device
    _check(q, "q", dtype, (B, H, N, d), dev)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, dtype, (B, Hkv, N, d), dev)
    if o is None:
        o = torch.empty((B, H, N, d), dtype=dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check(o, "o", dtype, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    if scale is None:
        scale = d ** -0.5
    heads = (B, H, Hkv) if gqa else (B, H)
    mask = (int(window[0]), int(window[1])) if window is not None else (int(bool(causal)),)
    st = getattr(library(), fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     *heads, N, d, float(scale), *mask,
                                     _stream(stream, q, k, v, o, lse))
    if st != 0:
        raise FAError(st, fn_name)
    return o, lse


def fa_forward(q, k, v, scale=None, causal=False, o=None, lse=None, stream=None):
    """O, lse = attention of bf16 [B,H,N,d] tensors (see fa_forward in fa.h)."""
    return _forward("fa_forward", q, k, v, scale, causal, o, lse, stream,
                    _torch().bfloat16)


def fa_forward_gqa(q, k, v, scale=None, causal=False, o=None, lse=None, stream=None):
    """Grouped-query forward: q [B,H,N,d], k and v [B,H_kv,N,d] bf16 with H_kv
    dividing H (see fa_forward_gqa in fa.h)."""
    return _forward("fa_forward_gqa", q, k, v, scale, causal, o, lse, stream,
                    _torch().bfloat16, gqa=True)


def fa_forward_window(q, k, v, window_left, window_right, scale=None, o=None, lse=None,
                      stream=None):
    """Local-window forward: key j visible to query i iff
    i - window_left <= j <= i + window_right (-1: no bound on that side); k, v
    may have fewer heads than q (see fa_forward_window in fa.h)."""
    return _forward("fa_forward_window", q, k, v, scale, None, o, lse, stream,
                    _torch().bfloat16, gqa=True, window=(window_left, window_right))


def fa_forward_f32(q, k, v, scale=None, causal=False, o=None, lse=None, stream=None):
    """fp32 in/out variant: inputs are rounded to bf16 as they are loaded."""
    return _forward("fa_forward_f32", q, k, v, scale, causal, o, lse, stream,
                    _torch().float32)


def _bwd_check(q, tensors, lse, outs, Hkv=None):
    """Checks [B,H,N,d] query-side tensors and [B,Hkv,N,d] K/V-side tensors
    (names k, v, dk, dv); allocates missing outputs."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    Hkv = H if Hkv is None else Hkv
    dev = q.device

    def shape_of(name):
        return (B, Hkv, N, d) if name in ("k", "v", "dk", "dv") else (B, H, N, d)

    for name, t in tensors:
        _check(t, name, torch.bfloat16, shape_of(name), dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, N), dev)
    res = []
    for name, t in outs:
        t = torch.empty(shape_of(name), dtype=torch.bfloat16, device=dev) if t is None else t
        _check(t, name, torch.bfloat16, shape_of(name), dev)
        res.append(t)
    return (B, H, N, d), dev, res


def _workspace(shape, dev, workspace):
    torch = _torch()
    need = fa_backward_workspace_size(*shape)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev:
        raise ValueError("workspace must be on the same device")
    return workspace, workspace.numel() * workspace.element_size()


def fa_backward(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
                workspace=None, stream=None):
    """dQ, dK, dV of sum(dout * O) (see fa_backward in fa.h)."""
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)))
    ws, ws_bytes = _workspace(shape, dev, workspace)
    scale = shape[3] ** -0.5 if scale is None else scale
    st = library().fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                               _ptr(dq), _ptr(dk), _ptr(dv), *shape, float(scale),
                               int(bool(causal)), _ptr(ws), ws_bytes,
                               _stream(stream, q, k, v, o, dout, lse, dq, dk, dv, ws))
    if st != 0:
        raise FAError(st, "fa_backward")
    return dq, dk, dv


def fa_backward_noalloc(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None,
                        dv=None, stream=None):
    """fa_backward with the row terms in the library's static scratch instead
    of a workspace (see fa_backward_noalloc in fa.h). The library allocates
    nothing; pass dq, dk, dv to keep this call free of torch allocations too."""
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)))
    scale = shape[3] ** -0.5 if scale is None else scale
    st = library().fa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                       _ptr(dq), _ptr(dk), _ptr(dv), *shape, float(scale),
                                       int(bool(causal)),
                                       _stream(stream, q, k, v, o, dout, lse, dq, dk, dv))
    if st != 0:
        raise FAError(st, "fa_backward_noalloc")
    return dq, dk, dv


def fa_backward_prep(o, dout, lse, workspace=None, stream=None):
    """Row terms (D_i = sum_k dout_ik O_ik, lse_i log2 e) into the workspace (see fa.h)."""
    shape, dev, _ = _bwd_check(o, (("o", o), ("dout", dout)), lse, ())
    ws, ws_bytes = _workspace(shape, dev, workspace)
    st = library().fa_backward_prep(_ptr(o), _ptr(dout), _ptr(lse), *shape, _ptr(ws), ws_bytes,
                                    _stream(stream, o, dout, lse, ws))
    if st != 0:
        raise FAError(st, "fa_backward_prep")
    return ws


def fa_backward_grads(q, k, v, dout, lse, workspace, scale=None, causal=False, dq=None,
                      dk=None, dv=None, stream=None):
    """dQ, dK, dV from the row terms fa_backward_prep left in `workspace` (see fa.h)."""
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)))
    if workspace is None or workspace.device != dev:
        raise ValueError("workspace from fa_backward_prep is required, on the same device")
    scale = shape[3] ** -0.5 if scale is None else scale
    st = library().fa_backward_grads(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                     _ptr(dq), _ptr(dk), _ptr(dv), *shape, float(scale),
                                     int(bool(causal)), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream, q, k, v, dout, lse, dq, dk, dv, workspace))
    if st != 0:
        raise FAError(st, "fa_backward_grads")
    return dq, dk, dv


def fa_backward_gqa(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
                    workspace=None, stream=None):
    """Grouped-query backward: dq [B,H,N,d]; dk, dv [B,H_kv,N,d], each the sum
    over its query heads (see fa_backward_gqa in fa.h)."""
    Hkv = _kv_heads(q, k)
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)), Hkv)
    ws, ws_bytes = _workspace(shape, dev, workspace)
    B, H, N, d = shape
    scale = d ** -0.5 if scale is None else scale
    st = library().fa_backward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d, float(scale),
                                   int(bool(causal)), _ptr(ws), ws_bytes,
                                   _stream(stream, q, k, v, o, dout, lse, dq, dk, dv, ws))
    if st != 0:
        raise FAError(st, "fa_backward_gqa")
    return dq, dk, dv


def fa_backward_grads_gqa(q, k, v, dout, lse, workspace, scale=None, causal=False, dq=None,
                          dk=None, dv=None, stream=None):
    """Second backward stage for grouped-query attention (see fa.h)."""
    Hkv = _kv_heads(q, k)
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)), Hkv)
    if workspace is None or workspace.device != dev:
        raise ValueError("workspace from fa_backward_prep is required, on the same device")
    B, H, N, d = shape
    scale = d ** -0.5 if scale is None else scale
    st = library().fa_backward_grads_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                         _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d,
                                         float(scale), int(bool(causal)), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _stream(stream, q, k, v, dout, lse, dq, dk, dv,
                                                 workspace))
    if st != 0:
        raise FAError(st, "fa_backward_grads_gqa")
    return dq, dk, dv


def fa_backward_window(q, k, v, o, dout, lse, window_left, window_right, scale=None, dq=None,
                       dk=None, dv=None, workspace=None, stream=None):
    """Local-window backward (see fa_backward_window in fa.h)."""
    Hkv = _kv_heads(q, k)
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)), Hkv)
    ws, ws_bytes = _workspace(shape, dev, workspace)
    B, H, N, d = shape
    scale = d ** -0.5 if scale is None else scale
    st = library().fa_backward_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                      _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d,
                                      float(scale), int(window_left), int(window_right),
                                      _ptr(ws), ws_bytes,
                                      _stream(stream, q, k, v, o, dout, lse, dq, dk, dv, ws))
    if st != 0:
        raise FAError(st, "fa_backward_window")
    return dq, dk, dv


def fa_backward_grads_window(q, k, v, dout, lse, workspace, window_left, window_right,
                             scale=None, dq=None, dk=None, dv=None, stream=None):
    """Second backward stage for local windows (see fa.h)."""
    Hkv = _kv_heads(q, k)
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)), Hkv)
    if workspace is None or workspace.device != dev:
        raise ValueError("workspace from fa_backward_prep is required, on the same device")
    B, H, N, d = shape
    scale = d ** -0.5 if scale is None else scale
    st = library().fa_backward_grads_window(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                            _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, N, d,
                                            float(scale), int(window_left), int(window_right),
                                            _ptr(workspace),
                                            workspace.numel() * workspace.element_size(),
                                            _stream(stream, q, k, v, dout, lse, dq, dk, dv,
                                                    workspace))
    if st != 0:
        raise FAError(st, "fa_backward_grads_window")
    return dq, dk, dv


# ---------------------------------------------------------------- block-sparse


def _block_mask(mask, B, H, N, dev):
    """The block mask as (tensor, head stride in bytes): uint8 or bool on the
    device, [nb, nb] shared by all heads (stride 0) or [B, H, nb, nb] one per
    query head, nb = ceil(N / 128), contiguous."""
    torch = _torch()
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    if mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError(f"block_mask: expected uint8 or bool, got {mask.dtype}")
    if tuple(mask.shape) == (nb, nb):
        stride = 0
    elif tuple(mask.shape) == (B, H, nb, nb):
        stride = nb * nb
    else:
        raise ValueError(f"block_mask: expected shape {(nb, nb)} or {(B, H, nb, nb)}, "
                         f"got {tuple(mask.shape)}")
    if not mask.is_contiguous():
        raise ValueError("block_mask must be contiguous")
    if mask.device != dev:
        raise ValueError(f"block_mask must be on {dev}")
    return mask, stride


def fa_forward_block_sparse(q, k, v, block_mask, window_left=-1, window_right=-1, scale=None,
                            o=None, lse=None, stream=None):
    """Block-sparse forward: blocks of 128 query rows x 128 keys whose mask
    byte is 0 are masked, on top of the window (-1, -1: none; -1, 0:
    causal); k, v may have fewer heads than q (see fa_forward_block_sparse
    in fa.h)."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(q, k)
    dev = q.device
    _check(q, "q", torch.bfloat16, (B, H, N, d), dev)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, torch.bfloat16, (B, Hkv, N, d), dev)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(o, "o", torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    bm, stride = _block_mask(block_mask, B, H, N, dev)
    scale = d ** -0.5 if scale is None else scale
    st = library().fa_forward_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                                           Hkv, N, d, float(scale), int(window_left),
                                           int(window_right), _ptr(bm), stride,
                                           _stream(stream, q, k, v, o, lse, bm))
    if st != 0:
        raise FAError(st, "fa_forward_block_sparse")
    return o, lse


def fa_backward_block_sparse(q, k, v, o, dout, lse, block_mask, window_left=-1,
                             window_right=-1, scale=None, dq=None, dk=None, dv=None,
                             workspace=None, stream=None):
    """Block-sparse backward, with the mask of the forward call (see
    fa_backward_block_sparse in fa.h)."""
    Hkv = _kv_heads(q, k)
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)), Hkv)
    ws, ws_bytes = _workspace(shape, dev, workspace)
    B, H, N, d = shape
    bm, stride = _block_mask(block_mask, B, H, N, dev)
    scale = d ** -0.5 if scale is None else scale
    st = library().fa_backward_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                            _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv,
                                            N, d, float(scale), int(window_left),
                                            int(window_right), _ptr(bm), stride, _ptr(ws),
                                            ws_bytes,
                                            _stream(stream, q, k, v, o, dout, lse, dq, dk, dv,
                                                    ws, bm))
    if st != 0:
        raise FAError(st, "fa_backward_block_sparse")
    return dq, dk, dv


def fa_backward_grads_block_sparse(q, k, v, dout, lse, workspace, block_mask, window_left=-1,
                                   window_right=-1, scale=None, dq=None, dk=None, dv=None,
                                   stream=None):
    """Second backward stage with a block-sparse mask (see fa.h)."""
    Hkv = _kv_heads(q, k)
    shape, dev, (dq, dk, dv) = _bwd_check(
        q, (("q", q), ("k", k), ("v", v), ("dout", dout)), lse,
        (("dq", dq), ("dk", dk), ("dv", dv)), Hkv)
    if workspace is None or workspace.device != dev:
        raise ValueError("workspace from fa_backward_prep is required, on the same device")
    B, H, N, d = shape
    bm, stride = _block_mask(block_mask, B, H, N, dev)
    scale = d ** -0.5 if scale is None else scale
    st = library().fa_backward_grads_block_sparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, H,
        Hkv, N, d, float(scale), int(window_left), int(window_right), _ptr(bm), stride,
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, q, k, v, dout, lse, dq, dk, dv, workspace, bm))
    if st != 0:
        raise FAError(st, "fa_backward_grads_block_sparse")
    return dq, dk, dv


# ---------------------------------------------------------------- FP8 forward

def fa_forward_fp8_workspace_size(B: int, H: int, H_kv: int, N: int, d: int) -> int:
    return int(library().fa_forward_fp8_workspace_size(B, H, H_kv, N, d))


def _signs_arg(signs, d):
    """Host int8 array for the C call (None: no rotation). Values are checked
    by the library (FA_ERR_ARG unless each is +1 or -1)."""
    if signs is None:
        return None, ctypes.c_void_p(0)
    vals = [int(x) for x in (signs.tolist() if hasattr(signs, "tolist") else signs)]
    if len(vals) != d:
        raise ValueError(f"signs: expected {d} values, got {len(vals)}")
    arr = (ctypes.c_int8 * d)(*[max(-128, min(127, x)) for x in vals])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def _fp8_shapes(q, k, v):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(q, k)
    dev = q.device
    _check(q, "q", torch.bfloat16, (B, H, N, d), dev)
    for name, t in (("k", k), ("v", v)):
        _check(t, name, torch.bfloat16, (B, Hkv, N, d), dev)
    return (B, H, Hkv, N, d), dev


def _fp8_workspace(shape, dev, workspace):
    torch = _torch()
    need = fa_forward_fp8_workspace_size(*shape)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev:
        raise ValueError("workspace must be on the same device")
    return workspace, workspace.numel() * workspace.element_size()


def fa_fp8_prepare(q, k, v, signs=None, workspace=None, stream=None):
    """Rotate (signs: d values of +1/-1, or None) and quantise q, k, v to e4m3
    into the FP8 workspace, returned as a uint8 tensor (layout in fa.h)."""
    shape, dev = _fp8_shapes(q, k, v)
    ws, ws_bytes = _fp8_workspace(shape, dev, workspace)
    keep, sp = _signs_arg(signs, shape[4])
    st = library().fa_fp8_prepare(_ptr(q), _ptr(k), _ptr(v), sp, *shape, _ptr(ws), ws_bytes,
                                  _stream(stream, q, k, v, ws))
    del keep
    if st != 0:
        raise FAError(st, "fa_fp8_prepare")
    return ws


def fa_forward_fp8_prepared(workspace, shape, scale=None, causal=False, o=None, lse=None,
                            stream=None):
    """Attention from a workspace fa_fp8_prepare filled; shape = (B, H, H_kv, N, d)."""
    torch = _torch()
    B, H, Hkv, N, d = (int(x) for x in shape)
    dev = workspace.device
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check(o, "o", torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    scale = d ** -0.5 if scale is None else scale
    st = library().fa_forward_fp8_prepared(_ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _ptr(o), _ptr(lse), B, H, Hkv, N, d, float(scale),
                                           int(bool(causal)), _stream(stream, workspace, o, lse))
    if st != 0:
        raise FAError(st, "fa_forward_fp8_prepared")
    return o, lse


def fa_forward_fp8(q, k, v, signs=None, scale=None, causal=False, o=None, lse=None,
                   workspace=None, stream=None):
    """FP8 forward with incoherent processing (see fa_forward_fp8 in fa.h):
    q [B,H,N,d], k and v [B,H_kv,N,d] bf16; signs: d values of +1/-1 (the
    random signs of the Hadamard rotation) or None for plain FP8."""
    torch = _torch()
    shape, dev = _fp8_shapes(q, k, v)
    B, H, Hkv, N, d = shape
    ws, ws_bytes = _fp8_workspace(shape, dev, workspace)
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check(o, "o", torch.bfloat16, (B, H, N, d), dev)
    _check(lse, "lse", torch.float32, (B, H, N), dev)
    scale = d ** -0.5 if scale is None else scale
    keep, sp = _signs_arg(signs, d)
    st = library().fa_forward_fp8(_ptr(q), _ptr(k), _ptr(v), sp, _ptr(o), _ptr(lse), *shape,
                                  float(scale), int(bool(causal)), _ptr(ws), ws_bytes,
                                  _stream(stream, q, k, v, o, lse, ws))
    del keep
    if st != 0:
        raise FAError(st, "fa_forward_fp8")
    return o, lse
