"""Python binding of libfa2.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
declared in ``include/fa2.h``; this module only checks tensor metadata,
allocates outputs with PyTorch (device memory and streams are PyTorch's) and
passes raw pointers.  There is no fallback: if ``libfa2.so`` is missing the
calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa2.so")

FA2_OK = 0
FA2_ERR_INVALID_ARGUMENT = 1
FA2_ERR_UNSUPPORTED = 2
FA2_ERR_HIP = 3

EXPORTS = ("fa2_fwd", "fa2_bwd", "fa2_bwd_stages", "fa2_fwd_f16", "fa2_bwd_f16", "fa2_bwd_stages_f16",
           "fa2_fwd_block_sparse", "fa2_bwd_block_sparse", "fa2_bwd_workspace_bytes",
           "fa2_bwd_stages_workspace_bytes", "fa2_validate_fwd", "fa2_validate_bwd", "fa2_status_string",
           "fa2_last_error", "fa2_bwd_noalloc", "fa2_fwd_block_sparse_f16", "fa2_bwd_block_sparse_f16",
           "fa2_fwd_olo", "fa2_bwd_olo", "fa2_bwd_stages_olo")
DTYPES = (torch.bfloat16, torch.float16)

BWD_PREPROCESS, BWD_MAIN, BWD_FINALIZE, BWD_ALL, BWD_DQ_ATOMIC = 1, 2, 4, 7, 8
NOALLOC_SCRATCH_BYTES = 16 << 20      # fa2_bwd_noalloc's static scratch per GPU
SPARSE_BLOCK = 128            # query rows and keys per block-sparse mask block
SPARSE_MAX_N = 262144

_lib = None


class FA2Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{status_string(status)}: {detail}")


def load(path: str | None = None):
    """Load libfa2.so (built in-tree by ``exact_io_aware_26_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_26_amd.build` "
                           "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa2_fwd.restype = i
    lib.fa2_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
    lib.fa2_bwd.restype = i
    lib.fa2_bwd_stages.argtypes = [ctypes.c_uint] + lib.fa2_bwd.argtypes
    lib.fa2_bwd_stages.restype = i
    lib.fa2_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa2_bwd_noalloc.restype = i
    lib.fa2_fwd_olo.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa2_fwd_olo.restype = i
    lib.fa2_bwd_olo.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
    lib.fa2_bwd_olo.restype = i
    lib.fa2_bwd_stages_olo.argtypes = [ctypes.c_uint] + lib.fa2_bwd_olo.argtypes
    lib.fa2_bwd_stages_olo.restype = i
    for name, like in (("fa2_fwd_f16", lib.fa2_fwd), ("fa2_bwd_f16", lib.fa2_bwd),
                       ("fa2_bwd_stages_f16", lib.fa2_bwd_stages)):
        fn = getattr(lib, name)
        fn.argtypes = like.argtypes
        fn.restype = i
    lib.fa2_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa2_fwd_block_sparse.restype = i
    lib.fa2_bwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                         i, i, i, i, i, i, f, vp]
    lib.fa2_bwd_block_sparse.restype = i
    for name, like in (("fa2_fwd_block_sparse_f16", lib.fa2_fwd_block_sparse),
                       ("fa2_bwd_block_sparse_f16", lib.fa2_bwd_block_sparse)):
        fn = getattr(lib, name)
        fn.argtypes = like.argtypes
        fn.restype = i
    lib.fa2_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa2_bwd_workspace_bytes.restype = sz
    lib.fa2_bwd_stages_workspace_bytes.argtypes = [ctypes.c_uint, i, i, i, i, i]
    lib.fa2_bwd_stages_workspace_bytes.restype = sz
    lib.fa2_validate_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f]
    lib.fa2_validate_fwd.restype = i
    lib.fa2_validate_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f]
    lib.fa2_validate_bwd.restype = i
    lib.fa2_status_string.argtypes = [i]
    lib.fa2_status_string.restype = ctypes.c_char_p
    lib.fa2_last_error.argtypes = []
    lib.fa2_last_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fa2_status_string(status).decode()


def _check(status: int, lib) -> None:
    if status != FA2_OK:
        raise FA2Error(status, lib.fa2_last_error().decode())


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream_handle(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dims(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, require_gpu: bool = True):
    """Check q, k, v and return (B, Hq, Hkv, N, d)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
    if q.dtype not in DTYPES:
        raise TypeError(f"q must be bfloat16 or float16, got {q.dtype}")
    if require_gpu and not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device {q.device}, got {t.device}")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return B, Hq, k.shape[1], N, d


def _check_tensor(name: str, t, dtype, shape, device) -> None:
    """A caller-supplied tensor: its dtype, shape, contiguity and device, checked before
    its pointer reaches the library (which can only check alignment and overlap)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on q's device {device}, got {t.device}")


def _check_o_lo(q, o_lo) -> None:
    if o_lo is not None:
        if q.dtype != torch.bfloat16:
            raise TypeError("o_lo is for bfloat16 tensors")
        _check_tensor("o_lo", o_lo, q.dtype, q.shape, q.device)


def check_forward_args(q, k, v, out=None, lse=None, require_gpu: bool = True, o_lo=None):
    """The metadata checks of ``forward``: returns (B, Hq, Hkv, N, d).  Raises TypeError
    or ValueError before anything is allocated or launched."""
    B, Hq, Hkv, N, d = _dims(q, k, v, require_gpu)
    if out is not None:
        _check_tensor("out", out, q.dtype, q.shape, q.device)
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, (B, Hq, N), q.device)
    _check_o_lo(q, o_lo)
    return B, Hq, Hkv, N, d


def check_backward_args(q, k, v, o, lse, do, workspace=None, grads=None, nbytes: int = 0,
                        require_gpu: bool = True, o_lo=None):
    """The metadata checks of ``backward``: returns (B, Hq, Hkv, N, d)."""
    B, Hq, Hkv, N, d = _dims(q, k, v, require_gpu)
    _check_tensor("o", o, q.dtype, q.shape, q.device)
    _check_o_lo(q, o_lo)
    _check_tensor("do", do, q.dtype, q.shape, q.device)
    _check_tensor("lse", lse, torch.float32, (B, Hq, N), q.device)
    if workspace is not None:
        _check_tensor("workspace", workspace, torch.uint8, None, q.device)
        if workspace.dim() != 1 or workspace.numel() < nbytes:
            raise ValueError(f"workspace must be a 1-D uint8 tensor of at least {nbytes} bytes")
    if grads is not None:
        if len(grads) != 3:
            raise ValueError("grads must be (dq, dk, dv)")
        for name, t, like in zip(("dq", "dk", "dv"), grads, (q, k, v)):
            _check_tensor(name, t, q.dtype, like.shape, q.device)
    return B, Hq, Hkv, N, d


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
            scale: float | None = None, out: torch.Tensor | None = None,
            lse: torch.Tensor | None = None, o_lo: torch.Tensor | None = None):
    """O = softmax(scale * q k^T [+ causal mask]) v and L (natural-log logsumexp per row).

    q [B,Hq,N,d], k/v [B,Hkv,N,d] contiguous GPU tensors, all bf16 or all f16.
    Returns (o [B,Hq,N,d] in q's dtype, lse [B,Hq,N] fp32).  scale defaults to
    1/sqrt(d).  ``o_lo`` (bf16 only): a tensor shaped like q that receives the
    rounding residual of o (fa2_fwd_olo), for ``backward(..., o_lo=...)``.
    """
    lib = load()
    B, Hq, Hkv, N, d = check_forward_args(q, k, v, out, lse, o_lo=o_lo)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if o_lo is not None:
        st = lib.fa2_fwd_olo(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(o_lo), _ptr(lse), B, Hq, Hkv,
                             N, d, int(bool(causal)), float(scale), _stream_handle(q))
    else:
        fwd = lib.fa2_fwd_f16 if q.dtype == torch.float16 else lib.fa2_fwd
        st = fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, N, d,
                 int(bool(causal)), float(scale), _stream_handle(q))
    _check(st, lib)
    return out, lse


def workspace_bytes(B: int, Hq: int, Hkv: int, N: int, d: int, stages: int = BWD_ALL) -> int:
    """Workspace bytes of a backward with these stage bits (the atomic-dQ mode needs more)."""
    return load().fa2_bwd_stages_workspace_bytes(int(stages), B, Hq, Hkv, N, d)


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             lse: torch.Tensor, do: torch.Tensor, causal: bool = False,
             scale: float | None = None, workspace: torch.Tensor | None = None,
             grads=None, stages: int = BWD_ALL, o_lo: torch.Tensor | None = None):
    """dQ, dK, dV of sum(do * o) for the forward above (P rebuilt from lse).

    Returns (dq [B,Hq,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d]) in q's dtype.  A caller
    may pass a reusable uint8 ``workspace`` of at least
    ``workspace_bytes(...)`` bytes (256-byte aligned), preallocated output
    tensors ``grads=(dq, dk, dv)``, and a subset of the launch ``stages``
    (issued in order; the workspace must carry over between partial calls).
    ``o_lo`` (bf16 only): the forward's rounding residual of o; D is then formed
    from o + o_lo (fa2_bwd_stages_olo).
    """
    lib = load()
    B, Hq, Hkv, N, d = _dims(q, k, v)
    nbytes = lib.fa2_bwd_stages_workspace_bytes(int(stages), B, Hq, Hkv, N, d)
    check_backward_args(q, k, v, o, lse, do, workspace, grads, nbytes, o_lo=o_lo)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k),
                                                  torch.empty_like(v))
    if o_lo is not None:
        st = lib.fa2_bwd_stages_olo(int(stages), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_lo), _ptr(lse),
                                    _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                    workspace.numel(), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                                    _stream_handle(q))
    else:
        bwd = lib.fa2_bwd_stages_f16 if q.dtype == torch.float16 else lib.fa2_bwd_stages
        st = bwd(int(stages), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                 B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _stream_handle(q))
    _check(st, lib)
    return dq, dk, dv


def backward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     lse: torch.Tensor, do: torch.Tensor, grads, causal: bool = False,
                     scale: float | None = None):
    """The bf16 backward through fa2_bwd_noalloc: no workspace, nothing allocated by the
    library or here; the caller passes the outputs ``grads=(dq, dk, dv)``.  Calls on
    one GPU share its static scratch and must not overlap in time."""
    lib = load()
    if q.dtype != torch.bfloat16:
        raise TypeError("fa2_bwd_noalloc takes bfloat16 tensors")
    B, Hq, Hkv, N, d = check_backward_args(q, k, v, o, lse, do, None, grads)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = grads
    st = lib.fa2_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                             _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
                             _stream_handle(q))
    _check(st, lib)
    return dq, dk, dv


def _block_mask(block_mask: torch.Tensor, N: int, device) -> torch.Tensor:
    """The mask as the library reads it: contiguous bytes [nb, nb] on q's device (bool is viewed, not copied)."""
    nb = (N + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    if block_mask.dtype != torch.uint8:
        raise TypeError(f"block_mask must be uint8 or bool, got {block_mask.dtype}")
    if tuple(block_mask.shape) != (nb, nb) or not block_mask.is_contiguous():
        raise ValueError(f"block_mask must be a contiguous [{nb}, {nb}] tensor, got {tuple(block_mask.shape)}")
    if block_mask.device != device:
        raise ValueError("block_mask must be on q's device")
    return block_mask


def forward_block_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: torch.Tensor,
                         causal: bool = False, scale: float | None = None,
                         out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Block-sparse forward (bf16 or f16): scores of 128 x 128 blocks whose mask byte is 0
    are masked.

    block_mask [ceil(N/128), ceil(N/128)] uint8 or bool on q's device, shared by every
    batch and head.  Rows with no unmasked key get o = 0 and lse = -inf.
    """
    lib = load()
    B, Hq, Hkv, N, d = check_forward_args(q, k, v, out, lse)
    bm = _block_mask(block_mask, N, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    fwd = lib.fa2_fwd_block_sparse_f16 if q.dtype == torch.float16 else lib.fa2_fwd_block_sparse
    st = fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(bm),
             B, Hq, Hkv, N, d, int(bool(causal)), float(scale), _stream_handle(q))
    _check(st, lib)
    return out, lse


def backward_block_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                          lse: torch.Tensor, do: torch.Tensor, block_mask: torch.Tensor,
                          causal: bool = False, scale: float | None = None,
                          workspace: torch.Tensor | None = None, grads=None):
    """Gradients of the block-sparse forward (same mask; o, lse from forward_block_sparse)."""
    lib = load()
    B, Hq, Hkv, N, d = _dims(q, k, v)
    bm = _block_mask(block_mask, N, q.device)
    nbytes = lib.fa2_bwd_workspace_bytes(B, Hq, Hkv, N, d)
    check_backward_args(q, k, v, o, lse, do, workspace, grads, nbytes)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k),
                                                  torch.empty_like(v))
    bwd = lib.fa2_bwd_block_sparse_f16 if q.dtype == torch.float16 else lib.fa2_bwd_block_sparse
    st = bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(bm), _ptr(workspace),
             workspace.numel(), B, Hq, Hkv, N, d, int(bool(causal)),
             float(scale), _stream_handle(q))
    _check(st, lib)
    return dq, dk, dv
