"""gated_pooling_amd -- Python binding of libcsa, the MI355X (gfx950) CSA/HCA
Compressor (THD-packed gated-softmax pooling), forward and backward.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libcsa.so`` (built in-tree by ``gated_pooling_amd.build``).  The
binding fails loudly if the library is missing; there is no CPU fallback.
PyTorch is used for device memory and the current stream.

Low level (same names and arguments as ``include/csa.h``, raw pointers):
  csa_compressor_total_comp, csa_compressor_check_support,
  csa_compressor_fwd_workspace_size, csa_compressor_bwd_workspace_size,
  csa_compressor_fwd, csa_compressor_bwd, csa_compressor_bwd_grads,
  csa_compressor_bwd_dape_reduce, csa_compressor_bwd_noalloc,
  csa_status_string, csa_last_error, csa_version

Tensor level:
  compressor_fwd(kv, score, ape, cu_seqlens, ratio, coff, total_comp, ...) -> out
  compressor_bwd(kv, score, ape, cu_seqlens, ratio, coff, total_comp, dout, ...)
      -> (dkv, dscore, dape)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

CSA_STATUS_SUCCESS = 0
CSA_STATUS_INVALID_VALUE = 1
CSA_STATUS_NOT_SUPPORTED = 2
CSA_STATUS_WORKSPACE_TOO_SMALL = 3
CSA_STATUS_LAUNCH_FAILED = 4
CSA_STATUS_DEVICE_ERROR = 5


class CsaError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {_status_name(status)}: {detail}")


class CsaNotSupported(CsaError, ValueError):
    """Outside the validated envelope (the pages' check_support raises
    ValueError for the same cases)."""


class CsaInvalidValue(CsaError, ValueError):
    pass


_lib = None


def lib():
    """Load libcsa.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m gated_pooling_amd.build` "
                               "or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        st = ctypes.c_int
        L.csa_status_string.restype = ctypes.c_char_p
        L.csa_status_string.argtypes = [st]
        L.csa_last_error.restype = ctypes.c_char_p
        L.csa_last_error.argtypes = []
        L.csa_version.restype = i32
        L.csa_version.argtypes = []
        L.csa_compressor_total_comp.restype = st
        L.csa_compressor_total_comp.argtypes = [P, i32, i32, P]
        L.csa_compressor_check_support.restype = st
        L.csa_compressor_check_support.argtypes = [i32, i32, i32, i32, i64, i64]
        for f in (L.csa_compressor_fwd_workspace_size, L.csa_compressor_bwd_workspace_size):
            f.restype = st
            f.argtypes = [i32, i32, i32, i32, i64, i64, P]
        L.csa_compressor_fwd.restype = st
        L.csa_compressor_fwd.argtypes = [P, P, P, P, P, i32, i64, i64, i32, i32, i32, P, P, sz, P]
        L.csa_compressor_bwd.restype = st
        L.csa_compressor_bwd.argtypes = [P, P, P, P, P, i32, i64, i64, i32, i32, i32, P, P, P, P, i32, P, sz, P]
        L.csa_compressor_bwd_grads.restype = st
        L.csa_compressor_bwd_grads.argtypes = [P, P, P, P, P, i32, i64, i64, i32, i32, i32, P, P, P, P, sz, P]
        L.csa_compressor_bwd_dape_reduce.restype = st
        L.csa_compressor_bwd_dape_reduce.argtypes = [i32, i32, i32, i32, i64, i64, P, P, sz, P]
        L.csa_compressor_bwd_noalloc.restype = st
        L.csa_compressor_bwd_noalloc.argtypes = [P, P, P, P, P, i32, i64, i64, i32, i32, i32, P, P, P, P, i32, P]
        _lib = L
    return _lib


def _status_name(status: int) -> str:
    try:
        return lib().csa_status_string(status).decode()
    except Exception:
        return f"status {status}"


def _check(status: int, func: str):
    if status == CSA_STATUS_SUCCESS:
        return
    detail = lib().csa_last_error().decode()
    cls = {CSA_STATUS_NOT_SUPPORTED: CsaNotSupported, CSA_STATUS_INVALID_VALUE: CsaInvalidValue}.get(status, CsaError)
    raise cls(status, func, detail)


# ---------------------------------------------------------------------------
# low level: the C entry points, raw pointers and sizes
# ---------------------------------------------------------------------------

def csa_status_string(status: int) -> str:
    return lib().csa_status_string(status).decode()


def csa_last_error() -> str:
    return lib().csa_last_error().decode()


def csa_version() -> int:
    return int(lib().csa_version())


def csa_compressor_total_comp(cu_seqlens_host, ratio: int) -> int:
    """total_comp from a host copy of cu_seqlens (sequence of ints or CPU int32 tensor)."""
    arr = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
    out = ctypes.c_int64(0)
    _check(lib().csa_compressor_total_comp(ctypes.cast(arr, ctypes.c_void_p), len(cu_seqlens_host) - 1, ratio,
                                           ctypes.byref(out)), "csa_compressor_total_comp")
    return int(out.value)


def csa_compressor_check_support(ratio, coff, head_dim, num_segments, total_tokens, total_comp) -> None:
    _check(lib().csa_compressor_check_support(ratio, coff, head_dim, num_segments, total_tokens, total_comp),
           "csa_compressor_check_support")


def csa_compressor_fwd_workspace_size(ratio, coff, head_dim, num_segments, total_tokens, total_comp) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().csa_compressor_fwd_workspace_size(ratio, coff, head_dim, num_segments, total_tokens, total_comp,
                                                   ctypes.byref(out)), "csa_compressor_fwd_workspace_size")
    return int(out.value)


def csa_compressor_bwd_workspace_size(ratio, coff, head_dim, num_segments, total_tokens, total_comp) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().csa_compressor_bwd_workspace_size(ratio, coff, head_dim, num_segments, total_tokens, total_comp,
                                                   ctypes.byref(out)), "csa_compressor_bwd_workspace_size")
    return int(out.value)


def csa_compressor_fwd(kv, score, ape, cu_seqlens, cu_seqlens_host, num_segments, total_tokens, total_comp, ratio,
                       coff, head_dim, out, workspace, workspace_bytes, stream) -> None:
    _check(lib().csa_compressor_fwd(kv, score, ape, cu_seqlens, cu_seqlens_host, num_segments, total_tokens,
                                    total_comp, ratio, coff, head_dim, out, workspace, workspace_bytes, stream),
           "csa_compressor_fwd")


def csa_compressor_bwd(kv, score, ape, cu_seqlens, cu_seqlens_host, num_segments, total_tokens, total_comp, ratio,
                       coff, head_dim, dout, dkv, dscore, dape, deterministic, workspace, workspace_bytes,
                       stream) -> None:
    _check(lib().csa_compressor_bwd(kv, score, ape, cu_seqlens, cu_seqlens_host, num_segments, total_tokens,
                                    total_comp, ratio, coff, head_dim, dout, dkv, dscore, dape, deterministic,
                                    workspace, workspace_bytes, stream), "csa_compressor_bwd")


def csa_compressor_bwd_grads(kv, score, ape, cu_seqlens, cu_seqlens_host, num_segments, total_tokens, total_comp,
                             ratio, coff, head_dim, dout, dkv, dscore, workspace, workspace_bytes, stream) -> None:
    _check(lib().csa_compressor_bwd_grads(kv, score, ape, cu_seqlens, cu_seqlens_host, num_segments, total_tokens,
                                          total_comp, ratio, coff, head_dim, dout, dkv, dscore, workspace,
                                          workspace_bytes, stream), "csa_compressor_bwd_grads")


def csa_compressor_bwd_dape_reduce(ratio, coff, head_dim, num_segments, total_tokens, total_comp, dape, workspace,
                                   workspace_bytes, stream) -> None:
    _check(lib().csa_compressor_bwd_dape_reduce(ratio, coff, head_dim, num_segments, total_tokens, total_comp, dape,
                                                workspace, workspace_bytes, stream),
           "csa_compressor_bwd_dape_reduce")


def csa_compressor_bwd_noalloc(kv, score, ape, cu_seqlens, cu_seqlens_host, num_segments, total_tokens, total_comp,
                               ratio, coff, head_dim, dout, dkv, dscore, dape, deterministic, stream) -> None:
    _check(lib().csa_compressor_bwd_noalloc(kv, score, ape, cu_seqlens, cu_seqlens_host, num_segments, total_tokens,
                                            total_comp, ratio, coff, head_dim, dout, dkv, dscore, dape,
                                            deterministic, stream), "csa_compressor_bwd_noalloc")


# ---------------------------------------------------------------------------
# tensor level
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream):
    """Context under which new tensors are allocated: the launch stream, so
    the caching allocator does not hand a block that the kernels still use
    to work on another stream when the local workspace is freed."""
    import contextlib
    torch = _torch()
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _dev(t, dtype, name, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _problem(kv, ape, cu_seqlens, ratio, coff):
    T, W = kv.shape
    if W % coff:
        raise ValueError("kv width must be coff * head_dim")
    return T, W // coff, cu_seqlens.numel() - 1


def workspace(nbytes: int, device):
    """A workspace tensor of at least nbytes (16-byte aligned)."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def host_cu(cu_seqlens_host):
    """A ctypes int32 array holding a host copy of cu_seqlens (or NULL)."""
    if cu_seqlens_host is None:
        return ctypes.c_void_p(0)
    vals = [int(x) for x in cu_seqlens_host]
    return (ctypes.c_int32 * len(vals))(*vals)


def compressor_fwd(kv, score, ape, cu_seqlens, ratio: int, coff: int, total_comp: int, out=None, ws=None,
                   stream=None, cu_seqlens_host=None):
    """out[total_comp, head_dim] (bf16).  cu_seqlens: int32 GPU tensor;
    cu_seqlens_host: optional host copy (list or CPU tensor) of the same."""
    torch = _torch()
    T, d, S = _problem(kv, ape, cu_seqlens, ratio, coff)
    W = coff * d
    nbytes = csa_compressor_fwd_workspace_size(ratio, coff, d, S, T, total_comp)
    with _on_stream(stream):
        if out is None:
            out = torch.empty(total_comp, d, dtype=torch.bfloat16, device=kv.device)
        if ws is None and nbytes:
            ws = workspace(nbytes, kv.device)
    csa_compressor_fwd(_dev(kv, torch.bfloat16, "kv", (T, W)), _dev(score, torch.bfloat16, "score", (T, W)),
                       _dev(ape, torch.float32, "ape", (ratio, W)), _dev(cu_seqlens, torch.int32, "cu_seqlens"),
                       host_cu(cu_seqlens_host), S, T, total_comp, ratio, coff, d, _dev(out, torch.bfloat16, "out", (total_comp, d)),
                       ctypes.c_void_p(ws.data_ptr() if ws is not None else 0),
                       ws.numel() if ws is not None else 0, _stream_ptr(stream))
    return out


def compressor_bwd(kv, score, ape, cu_seqlens, ratio: int, coff: int, total_comp: int, dout, dkv=None,
                   dscore=None, dape=None, ws=None, stream=None, deterministic: int = 1, cu_seqlens_host=None):
    """(dkv, dscore, dape): bf16 [T, coff*d] x2 (fully written), fp32 [ratio, coff*d]."""
    torch = _torch()
    T, d, S = _problem(kv, ape, cu_seqlens, ratio, coff)
    W = coff * d
    nbytes = csa_compressor_bwd_workspace_size(ratio, coff, d, S, T, total_comp)
    with _on_stream(stream):
        if dkv is None:
            dkv = torch.empty(T, W, dtype=torch.bfloat16, device=kv.device)
        if dscore is None:
            dscore = torch.empty(T, W, dtype=torch.bfloat16, device=kv.device)
        if dape is None:
            dape = torch.empty(ratio, W, dtype=torch.float32, device=kv.device)
        if ws is None:
            ws = workspace(nbytes, kv.device)
    csa_compressor_bwd(_dev(kv, torch.bfloat16, "kv", (T, W)), _dev(score, torch.bfloat16, "score", (T, W)),
                       _dev(ape, torch.float32, "ape", (ratio, W)), _dev(cu_seqlens, torch.int32, "cu_seqlens"),
                       host_cu(cu_seqlens_host), S, T, total_comp, ratio, coff, d, _dev(dout, torch.bfloat16, "dout", (total_comp, d)),
                       _dev(dkv, torch.bfloat16, "dkv", (T, W)), _dev(dscore, torch.bfloat16, "dscore", (T, W)),
                       _dev(dape, torch.float32, "dape", (ratio, W)), deterministic,
                       ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_ptr(stream))
    return dkv, dscore, dape
