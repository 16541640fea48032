"""Exact attention for AMD Instinct MI355X (gfx950): Python binding of libfa.so.

The binding only marshals arguments: it checks torch tensors (dtype, shape,
contiguity, device), passes their device pointers and the current HIP stream to
the C ABI declared in include/fa.h, and turns error codes into exceptions.
Every step of the computation runs in the library's HIP kernels; there is no
fallback of any kind -- if libfa.so is missing or fails to load, calls raise.

    import torch, io_aware_exact_02_amd as fa
    O, lse = fa.forward(q, k, v, causal=True)                # q,k,v: [B,H,T,d] bf16/fp32
    dQ, dK, dV = fa.backward(q, k, v, O, dO, lse, causal=True)

The lower-level names mirror the C entry points one to one (fa_fwd, fa_bwd,
fa_bwd_workspace_bytes, fa_strerror) and write into caller-provided outputs.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FA_F32", "FA_BF16", "FA_BWD_PRE", "FA_BWD_MAIN", "FA_BWD_POST", "FA_BWD_ALL", "FAError", "LIB_PATH", "library", "fa_fwd", "fa_bwd",
    "fa_bwd_phases", "fa_bwd_workspace_bytes", "fa_strerror", "fa_abi_version", "forward", "backward",
    "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes", "forward_splitkv", "fa_fwd_masked", "fa_bwd_masked",
    "fa_bwd_masked_phases", "forward_masked", "backward_masked", "MASK_BLOCK", "fa_fwd_window", "fa_bwd_window",
    "fa_bwd_window_phases", "forward_window", "backward_window", "fa_fwd_docs", "fa_bwd_docs",
    "fa_bwd_docs_phases", "forward_docs", "backward_docs", "EXPORTED_SYMBOLS", "fa_bwd_noalloc",
    "NOALLOC_SCRATCH_BYTES",
]

FA_F32 = 0
FA_BF16 = 1
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
EXPORTED_SYMBOLS = ("fa_fwd", "fa_bwd", "fa_bwd_phases", "fa_bwd_workspace_bytes", "fa_strerror",
                    "fa_abi_version", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_bytes", "fa_fwd_masked",
                    "fa_bwd_masked", "fa_bwd_masked_phases", "fa_fwd_window", "fa_bwd_window",
                    "fa_bwd_window_phases", "fa_fwd_docs", "fa_bwd_docs", "fa_bwd_docs_phases",
                    "fa_bwd_noalloc")
NOALLOC_SCRATCH_BYTES = 16 << 20   # FA_NOALLOC_SCRATCH_BYTES: fa_bwd_noalloc's fixed workspace
MASK_BLOCK = 128          # block-mask granularity, in query rows and in keys
FA_BWD_PRE, FA_BWD_MAIN, FA_BWD_POST, FA_BWD_ALL = 1, 2, 4, 7

_lib = None


class FAError(RuntimeError):
    """A non-zero fa_status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_strerror(status)} (fa_status {status})")


def library() -> ctypes.CDLL:
    """Load libfa.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m io_aware_exact_02_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_phases.argtypes = lib.fa_bwd.argtypes[:-1] + [i, vp]
    lib.fa_bwd_phases.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp, sz, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_masked.argtypes = lib.fa_fwd.argtypes[:-1] + [vp, i, vp]
    lib.fa_fwd_masked.restype = i
    lib.fa_bwd_masked.argtypes = lib.fa_bwd.argtypes[:19] + [vp, i, vp, sz, vp]
    lib.fa_bwd_masked.restype = i
    lib.fa_bwd_masked_phases.argtypes = lib.fa_bwd.argtypes[:19] + [vp, i, vp, sz, i, vp]
    lib.fa_bwd_masked_phases.restype = i
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp]
    lib.fa_fwd_window.restype = i
    lib.fa_bwd_window.argtypes = [vp] * 9 + [i, i, i, i, i, f, i, i, i, i, i, vp, sz, vp]
    lib.fa_bwd_window.restype = i
    lib.fa_bwd_window_phases.argtypes = lib.fa_bwd_window.argtypes[:-1] + [i, vp]
    lib.fa_bwd_window_phases.restype = i
    lib.fa_fwd_docs.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, i, i, vp]
    lib.fa_fwd_docs.restype = i
    lib.fa_bwd_docs.argtypes = [vp] * 9 + [i, i, i, i, f, i, vp, i, i, i, i, vp, sz, vp]
    lib.fa_bwd_docs.restype = i
    lib.fa_bwd_docs_phases.argtypes = lib.fa_bwd_docs.argtypes[:-1] + [i, vp]
    lib.fa_bwd_docs_phases.restype = i
    lib.fa_bwd_noalloc.argtypes = lib.fa_bwd.argtypes[:19] + [vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_splitkv_workspace_bytes.restype = sz
    _lib = lib
    return lib


def fa_strerror(status: int) -> str:
    return library().fa_strerror(int(status)).decode()


def fa_abi_version() -> int:
    return int(library().fa_abi_version())


def fa_bwd_workspace_bytes(B, H, Tq, Tk, d, dtype, grad_dtype) -> int:
    return int(library().fa_bwd_workspace_bytes(B, H, Tq, Tk, d, dtype, grad_dtype))


# ----------------------------------------------------------------------------------
# torch marshalling
# ----------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _check(t, name, shape, dtype=None, device=None):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def _stream_handle(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def fa_fwd(q, k, v, o, lse, *, scale=None, causal=False, stream=None) -> None:
    """Launch the forward pass into caller-provided `o` [B,H,Tq,d] and `lse` [B,H,Tq] fp32.

    `o` has the inputs' dtype, or float32 for bf16 inputs (O left unrounded)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    dev = q.device
    _check(q, "q", (B, H, Tq, d), device=dev)
    _check(k, "k", (B, H, Tk, d), q.dtype, dev)
    _check(v, "v", (B, H, Tk, d), q.dtype, dev)
    _check(o, "o", (B, H, Tq, d), None, dev)
    _check(lse, "lse", (B, H, Tq), torch.float32, dev)
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          B, H, Tq, Tk, d, c, int(bool(causal)), _dtype_code(q), _dtype_code(o),
                          _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_fwd")


def fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, d, nsplit=0) -> int:
    return int(library().fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, d, nsplit))


def fa_fwd_splitkv(q, k, v, o, lse, workspace, *, scale=None, causal=False, nsplit=0, stream=None) -> None:
    """Split-key forward (bf16 inputs, few query rows) into caller-provided `o`, `lse`;
    `workspace` is a uint8 device tensor of fa_fwd_splitkv_workspace_bytes(...) bytes."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    dev = q.device
    _check(q, "q", (B, H, Tq, d), device=dev)
    _check(k, "k", (B, H, Tk, d), q.dtype, dev)
    _check(v, "v", (B, H, Tk, d), q.dtype, dev)
    _check(o, "o", (B, H, Tq, d), None, dev)
    _check(lse, "lse", (B, H, Tq), torch.float32, dev)
    _check(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = library().fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, Tq, Tk, d, c, int(bool(causal)), _dtype_code(q), _dtype_code(o),
                                  int(nsplit), workspace.data_ptr(), workspace.numel(),
                                  _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_fwd_splitkv")


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, workspace, *, scale=None, causal=False, stream=None) -> None:
    """Launch the backward pass into caller-provided dq, dk, dv (bf16 or fp32).

    `workspace` is a uint8 GPU tensor of at least fa_bwd_workspace_bytes(...) bytes.
    """
    fa_bwd_phases(q, k, v, o, do, lse, dq, dk, dv, workspace, FA_BWD_ALL, scale=scale, causal=causal,
                  stream=stream)


def fa_bwd_phases(q, k, v, o, do, lse, dq, dk, dv, workspace, phases, *, scale=None, causal=False,
                  stream=None) -> None:
    """Launch the named backward phases (an OR of FA_BWD_PRE, FA_BWD_MAIN, FA_BWD_POST)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    dev = q.device
    _check(q, "q", (B, H, Tq, d), device=dev)
    for name, t, T in (("k", k, Tk), ("v", v, Tk), ("do", do, Tq)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    _check(o, "o", (B, H, Tq, d), None, dev)
    _check(lse, "lse", (B, H, Tq), torch.float32, dev)
    _check(dq, "dq", (B, H, Tq, d), None, dev)
    _check(dk, "dk", (B, H, Tk, d), dq.dtype, dev)
    _check(dv, "dv", (B, H, Tk, d), dq.dtype, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    st = library().fa_bwd_phases(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Tq, Tk, d, c,
                                 int(bool(causal)), _dtype_code(q), _dtype_code(o), _dtype_code(dq),
                                 workspace.data_ptr(), nbytes,
                                 int(phases), _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_bwd_phases")


def fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, *, scale=None, causal=False, stream=None) -> None:
    """The backward pass with no workspace argument (fa_bwd_noalloc): the library's
    fixed per-GPU scratch holds the row terms, so the call allocates nothing.
    Problems whose workspace would exceed NOALLOC_SCRATCH_BYTES raise FAError
    (FA_ERR_SCRATCH); calls that overlap on one GPU race on the shared scratch."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    dev = q.device
    _check(q, "q", (B, H, Tq, d), device=dev)
    for name, t, T in (("k", k, Tk), ("v", v, Tk), ("do", do, Tq)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    _check(o, "o", (B, H, Tq, d), None, dev)
    _check(lse, "lse", (B, H, Tq), torch.float32, dev)
    _check(dq, "dq", (B, H, Tq, d), None, dev)
    _check(dk, "dk", (B, H, Tk, d), dq.dtype, dev)
    _check(dv, "dv", (B, H, Tk, d), dq.dtype, dev)
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = library().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Tq, Tk, d, c,
                                  int(bool(causal)), _dtype_code(q), _dtype_code(o), _dtype_code(dq),
                                  _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_bwd_noalloc")


def _check_mask(block_mask, H, Tq, Tk, dev):
    torch = _torch()
    nqb, nkb = -(-Tq // MASK_BLOCK), -(-Tk // MASK_BLOCK)
    if block_mask.dim() != 3 or block_mask.shape[0] not in (1, H):
        raise ValueError(f"block_mask: expected shape (1 or {H}, {nqb}, {nkb}), got {tuple(block_mask.shape)}")
    _check(block_mask, "block_mask", (block_mask.shape[0], nqb, nkb), torch.uint8, dev)
    return int(block_mask.shape[0])


def fa_fwd_masked(q, k, v, o, lse, block_mask, *, scale=None, causal=False, stream=None) -> None:
    """Block-sparse forward (bf16 inputs) into caller-provided `o`, `lse`.

    `block_mask`: uint8 GPU tensor [1 or H, ceil(Tq/128), ceil(Tk/128)]; a non-zero
    entry keeps that (128-query, 128-key) tile."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    dev = q.device
    _check(q, "q", (B, H, Tq, d), device=dev)
    _check(k, "k", (B, H, Tk, d), q.dtype, dev)
    _check(v, "v", (B, H, Tk, d), q.dtype, dev)
    _check(o, "o", (B, H, Tq, d), None, dev)
    _check(lse, "lse", (B, H, Tq), torch.float32, dev)
    mh = _check_mask(block_mask, H, Tq, Tk, dev)
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = library().fa_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 B, H, Tq, Tk, d, c, int(bool(causal)), _dtype_code(q), _dtype_code(o),
                                 block_mask.data_ptr(), mh, _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_fwd_masked")


def fa_bwd_masked(q, k, v, o, do, lse, dq, dk, dv, block_mask, workspace, *, scale=None, causal=False,
                  stream=None) -> None:
    """Block-sparse backward (bf16 inputs, d in {64, 128, 256}) into caller-provided dq, dk, dv."""
    fa_bwd_masked_phases(q, k, v, o, do, lse, dq, dk, dv, block_mask, workspace, FA_BWD_ALL, scale=scale,
                         causal=causal, stream=stream)


def fa_bwd_masked_phases(q, k, v, o, do, lse, dq, dk, dv, block_mask, workspace, phases, *, scale=None,
                         causal=False, stream=None) -> None:
    """The named phases of the block-sparse backward (an OR of FA_BWD_PRE, _MAIN, _POST)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    dev = q.device
    _check(q, "q", (B, H, Tq, d), device=dev)
    for name, t, T in (("k", k, Tk), ("v", v, Tk), ("do", do, Tq)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    _check(o, "o", (B, H, Tq, d), None, dev)
    _check(lse, "lse", (B, H, Tq), torch.float32, dev)
    _check(dq, "dq", (B, H, Tq, d), None, dev)
    _check(dk, "dk", (B, H, Tk, d), dq.dtype, dev)
    _check(dv, "dv", (B, H, Tk, d), dq.dtype, dev)
    mh = _check_mask(block_mask, H, Tq, Tk, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    st = library().fa_bwd_masked_phases(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Tq, Tk,
                                        d, c, int(bool(causal)), _dtype_code(q), _dtype_code(o), _dtype_code(dq),
                                        block_mask.data_ptr(), mh, workspace.data_ptr(), nbytes, int(phases),
                                        _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_bwd_masked_phases")


def _window(window):
    wl, wr = (int(x) for x in window)
    return wl, wr


def fa_fwd_window(q, k, v, o, lse, window, *, scale=None, stream=None) -> None:
    """Sliding-window forward (bf16 inputs): key l is visible from query r iff
    r - window[0] <= l <= r + window[1] (-1 = unbounded side)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    dev = q.device
    _check(q, "q", (B, H, Tq, d), device=dev)
    _check(k, "k", (B, H, Tk, d), q.dtype, dev)
    _check(v, "v", (B, H, Tk, d), q.dtype, dev)
    _check(o, "o", (B, H, Tq, d), None, dev)
    _check(lse, "lse", (B, H, Tq), torch.float32, dev)
    wl, wr = _window(window)
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = library().fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 B, H, Tq, Tk, d, c, wl, wr, _dtype_code(q), _dtype_code(o),
                                 _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_fwd_window")


def fa_bwd_window(q, k, v, o, do, lse, dq, dk, dv, window, workspace, *, scale=None, stream=None) -> None:
    """Sliding-window backward (bf16 inputs) into caller-provided dq, dk, dv."""
    fa_bwd_window_phases(q, k, v, o, do, lse, dq, dk, dv, window, workspace, FA_BWD_ALL, scale=scale,
                         stream=stream)


def fa_bwd_window_phases(q, k, v, o, do, lse, dq, dk, dv, window, workspace, phases, *, scale=None,
                         stream=None) -> None:
    """The named phases of the sliding-window backward (an OR of FA_BWD_PRE, _MAIN, _POST)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    dev = q.device
    _check(q, "q", (B, H, Tq, d), device=dev)
    for name, t, T in (("k", k, Tk), ("v", v, Tk), ("do", do, Tq)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    _check(o, "o", (B, H, Tq, d), None, dev)
    _check(lse, "lse", (B, H, Tq), torch.float32, dev)
    _check(dq, "dq", (B, H, Tq, d), None, dev)
    _check(dk, "dk", (B, H, Tk, d), dq.dtype, dev)
    _check(dv, "dv", (B, H, Tk, d), dq.dtype, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    wl, wr = _window(window)
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    st = library().fa_bwd_window_phases(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Tq, Tk,
                                        d, c, wl, wr, _dtype_code(q), _dtype_code(o), _dtype_code(dq),
                                        workspace.data_ptr(), nbytes, int(phases), _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_bwd_window_phases")


def _check_docs(cu_seqlens, dev):
    torch = _torch()
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError(f"cu_seqlens: expected shape (ndocs + 1,) with ndocs >= 1, got {tuple(cu_seqlens.shape)}")
    _check(cu_seqlens, "cu_seqlens", tuple(cu_seqlens.shape), torch.int32, dev)
    return int(cu_seqlens.numel()) - 1


def fa_fwd_docs(q, k, v, o, lse, cu_seqlens, *, scale=None, causal=False, stream=None) -> None:
    """Document-masked forward (bf16 inputs) of packed sequences [B, H, T, d]: query r
    sees key l iff both lie in one document (and l <= r when causal).  `cu_seqlens`:
    int32 GPU tensor [ndocs + 1] of offsets, 0 first and T last, shared by all (B, H);
    its values are read on the device only."""
    torch = _torch()
    B, H, T, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    _check(o, "o", (B, H, T, d), None, dev)
    _check(lse, "lse", (B, H, T), torch.float32, dev)
    nd = _check_docs(cu_seqlens, dev)
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = library().fa_fwd_docs(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               B, H, T, d, c, int(bool(causal)), cu_seqlens.data_ptr(), nd, _dtype_code(q),
                               _dtype_code(o), _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_fwd_docs")


def fa_bwd_docs(q, k, v, o, do, lse, dq, dk, dv, cu_seqlens, workspace, *, scale=None, causal=False,
                stream=None) -> None:
    """Document-masked backward (bf16 inputs) into caller-provided dq, dk, dv."""
    fa_bwd_docs_phases(q, k, v, o, do, lse, dq, dk, dv, cu_seqlens, workspace, FA_BWD_ALL, scale=scale,
                       causal=causal, stream=stream)


def fa_bwd_docs_phases(q, k, v, o, do, lse, dq, dk, dv, cu_seqlens, workspace, phases, *, scale=None,
                       causal=False, stream=None) -> None:
    """The named phases of the document-masked backward (an OR of FA_BWD_PRE, _MAIN, _POST)."""
    torch = _torch()
    B, H, T, d = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _check(t, name, (B, H, T, d), q.dtype, dev)
    _check(o, "o", (B, H, T, d), None, dev)
    _check(lse, "lse", (B, H, T), torch.float32, dev)
    _check(dq, "dq", (B, H, T, d), None, dev)
    _check(dk, "dk", (B, H, T, d), dq.dtype, dev)
    _check(dv, "dv", (B, H, T, d), dq.dtype, dev)
    nd = _check_docs(cu_seqlens, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    c = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = workspace.numel() * workspace.element_size()
    st = library().fa_bwd_docs_phases(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, T, d, c,
                                      int(bool(causal)), cu_seqlens.data_ptr(), nd, _dtype_code(q), _dtype_code(o),
                                      _dtype_code(dq), workspace.data_ptr(), nbytes, int(phases),
                                      _stream_handle(stream, dev))
    if st != 0:
        raise FAError(st, "fa_bwd_docs_phases")


def forward(q, k, v, *, causal=False, scale=None, out_dtype=None, stream=None):
    """Allocate O and lse with torch and run fa_fwd.  Returns (O, lse).

    out_dtype: O's dtype (default: the inputs'; torch.float32 allowed for bf16)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    o = torch.empty(q.shape, dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, stream=stream)
    return o, lse


def forward_splitkv(q, k, v, *, causal=False, scale=None, out_dtype=None, nsplit=0, stream=None):
    """Allocate O, lse and the partials' workspace with torch and run fa_fwd_splitkv."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    o = torch.empty(q.shape, dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    nbytes = fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, d, nsplit)
    if nbytes == 0:
        raise ValueError("invalid arguments for fa_fwd_splitkv")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    fa_fwd_splitkv(q, k, v, o, lse, ws, scale=scale, causal=causal, nsplit=nsplit, stream=stream)
    return o, lse


def backward(q, k, v, o, do, lse, *, causal=False, scale=None, grad_dtype=None, stream=None):
    """Allocate gradients and workspace with torch and run fa_bwd.  Returns (dQ, dK, dV).

    grad_dtype defaults to the input dtype (torch.float32 is also allowed for
    bf16 inputs).
    """
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    gd = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty((B, H, Tq, d), dtype=gd, device=q.device)
    dk = torch.empty((B, H, Tk, d), dtype=gd, device=q.device)
    dv = torch.empty((B, H, Tk, d), dtype=gd, device=q.device)
    nbytes = fa_bwd_workspace_bytes(B, H, Tq, Tk, d, _dtype_code(q), _dtype_code(dq))
    if nbytes == 0:
        raise ValueError("invalid arguments for fa_bwd")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=scale, causal=causal, stream=stream)
    return dq, dk, dv


def forward_masked(q, k, v, block_mask, *, causal=False, scale=None, out_dtype=None, stream=None):
    """Allocate O and lse with torch and run fa_fwd_masked.  Returns (O, lse)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    o = torch.empty(q.shape, dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    fa_fwd_masked(q, k, v, o, lse, block_mask, scale=scale, causal=causal, stream=stream)
    return o, lse


def backward_masked(q, k, v, o, do, lse, block_mask, *, causal=False, scale=None, grad_dtype=None, stream=None):
    """Allocate gradients and workspace with torch and run fa_bwd_masked.  Returns (dQ, dK, dV)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    gd = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty((B, H, Tq, d), dtype=gd, device=q.device)
    dk = torch.empty((B, H, Tk, d), dtype=gd, device=q.device)
    dv = torch.empty((B, H, Tk, d), dtype=gd, device=q.device)
    nbytes = fa_bwd_workspace_bytes(B, H, Tq, Tk, d, _dtype_code(q), _dtype_code(dq))
    if nbytes == 0:
        raise ValueError("invalid arguments for fa_bwd_masked")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    fa_bwd_masked(q, k, v, o, do, lse, dq, dk, dv, block_mask, ws, scale=scale, causal=causal, stream=stream)
    return dq, dk, dv


def forward_window(q, k, v, window, *, scale=None, out_dtype=None, stream=None):
    """Allocate O and lse with torch and run fa_fwd_window.  Returns (O, lse)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    o = torch.empty(q.shape, dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    fa_fwd_window(q, k, v, o, lse, window, scale=scale, stream=stream)
    return o, lse


def backward_window(q, k, v, o, do, lse, window, *, scale=None, grad_dtype=None, stream=None):
    """Allocate gradients and workspace with torch and run fa_bwd_window.  Returns (dQ, dK, dV)."""
    torch = _torch()
    B, H, Tq, d = q.shape
    Tk = k.shape[2]
    gd = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty((B, H, Tq, d), dtype=gd, device=q.device)
    dk = torch.empty((B, H, Tk, d), dtype=gd, device=q.device)
    dv = torch.empty((B, H, Tk, d), dtype=gd, device=q.device)
    nbytes = fa_bwd_workspace_bytes(B, H, Tq, Tk, d, _dtype_code(q), _dtype_code(dq))
    if nbytes == 0:
        raise ValueError("invalid arguments for fa_bwd_window")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    fa_bwd_window(q, k, v, o, do, lse, dq, dk, dv, window, ws, scale=scale, stream=stream)
    return dq, dk, dv


def forward_docs(q, k, v, cu_seqlens, *, causal=False, scale=None, out_dtype=None, stream=None):
    """Allocate O and lse with torch and run fa_fwd_docs.  Returns (O, lse)."""
    torch = _torch()
    B, H, T, d = q.shape
    o = torch.empty(q.shape, dtype=q.dtype if out_dtype is None else out_dtype, device=q.device)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    fa_fwd_docs(q, k, v, o, lse, cu_seqlens, scale=scale, causal=causal, stream=stream)
    return o, lse


def backward_docs(q, k, v, o, do, lse, cu_seqlens, *, causal=False, scale=None, grad_dtype=None, stream=None):
    """Allocate gradients and workspace with torch and run fa_bwd_docs.  Returns (dQ, dK, dV)."""
    torch = _torch()
    B, H, T, d = q.shape
    gd = q.dtype if grad_dtype is None else grad_dtype
    dq = torch.empty((B, H, T, d), dtype=gd, device=q.device)
    dk = torch.empty((B, H, T, d), dtype=gd, device=q.device)
    dv = torch.empty((B, H, T, d), dtype=gd, device=q.device)
    nbytes = fa_bwd_workspace_bytes(B, H, T, T, d, _dtype_code(q), _dtype_code(dq))
    if nbytes == 0:
        raise ValueError("invalid arguments for fa_bwd_docs")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    fa_bwd_docs(q, k, v, o, do, lse, dq, dk, dv, cu_seqlens, ws, scale=scale, causal=causal, stream=stream)
    return dq, dk, dv
