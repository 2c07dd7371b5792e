"""ctypes binding of libh3attn.so (the HIP kernels and their C ABI).

Argument marshalling only: dtype/device/shape checks, raw device pointers and the current HIP
stream go to the C ABI, and every step runs in the library's kernels. There is no fallback
path: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libh3attn.so")

STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "LAUNCH"}

# (name, restype, argtypes) of every exported symbol declared in include/h3attn.h
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class Grid(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]


SIGNATURES = {
    "h3attn_version": (ctypes.c_char_p, []),
    "h3attn_last_error": (ctypes.c_char_p, []),
    "h3attn_keep_count": (_I32, [_I32, ctypes.c_double]),
    "h3attn_select_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I64, _I32, _I32]),
    "h3attn_qk_norm_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, Grid,
                                           _I32, _I32, _I32, ctypes.c_float, ctypes.c_float, _P]),
    "h3attn_qk_norm_rope_pool": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, Grid,
                                                _I32, _I32, _I32, ctypes.c_float, ctypes.c_float, _I32,
                                                _P, ctypes.c_size_t, _P]),
    "h3attn_subblock_select_pooled": (ctypes.c_int, [_I32, _I32, _I64, _I32, _I32, ctypes.c_double,
                                                     _I32, _P, _P, ctypes.c_size_t, _P]),
    "h3attn_dense_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _P]),
    "h3attn_subblock_select": (ctypes.c_int, [_P, _P, _I32, _I32, _I64, _I32, _I32, ctypes.c_double,
                                              _I32, _P, _P, ctypes.c_size_t, _P]),
    "h3attn_block_sparse_fwd": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I64, _I32,
                                               _I32, _P]),
    "h3attn_block_sparse_grouped_fwd": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I64, _I32,
                                                       _I32, _I32, _P]),
    "h3attn_threshold_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I64, _I32, _I32]),
    "h3attn_subblock_threshold_count": (ctypes.c_int, [_P, _P, _I32, _I32, _I64, _I32, _I32, ctypes.c_double,
                                                       _P, _P, ctypes.c_size_t, _P]),
    "h3attn_subblock_threshold_fill": (ctypes.c_int, [_I32, _I32, _I64, _I32, _I32, _P, _P, _I64, _P,
                                                      ctypes.c_size_t, _P]),
    "h3attn_block_sparse_csr_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _I32,
                                                   _P]),
    "h3attn_block_sparse_csr_grouped_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I32,
                                                           _I32, _I32, _P]),
    "h3attn_check_block_idx": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P]),
    "h3attn_check_csr": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _P, _P]),
    "h3attn_adaln_modulate": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I32, ctypes.c_float, _P]),
    "h3attn_swiglu": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I64, _I64, _P]),
    "h3attn_residual_workspace_bytes": (ctypes.c_size_t, [_I64]),
    "h3attn_residual_change": (ctypes.c_int, [_P, _P, _I64, _P, _P, ctypes.c_size_t, _P]),
    "h3attn_residual_change_noalloc": (ctypes.c_int, [_P, _P, _I64, _P, _P]),
    "h3attn_cache_gate_init": (ctypes.c_int, [_P, ctypes.c_double, _I32]),
    "h3attn_cache_gate_decide": (_I32, [_P, ctypes.c_double]),
    "h3attn_cache_gate_decide_sums": (_I32, [_P, _P]),
    "h3attn_fp8_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I64, _I32, _I32]),
    "h3attn_fp8_quantize": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _I32,
                                           _P, ctypes.c_size_t, _P]),
    "h3attn_fp8_dense_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _I32, _P]),
    "h3attn_fp8_block_sparse_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I64,
                                                   _I32, _I32, _I32, _P]),
}


class CacheGateState(ctypes.Structure):
    _fields_ = [("threshold", ctypes.c_double), ("max_consecutive", ctypes.c_int32),
                ("consecutive", ctypes.c_int32), ("steps", ctypes.c_int64)]


class H3AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"h3attn {STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libh3attn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950); there is no non-HIP fallback")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise H3AttnError(status, load_library().h3attn_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _need_shape(t: torch.Tensor, name: str, shape, like: torch.Tensor):
    """t has exactly `shape` and lives on the same device as `like` (the kernels write and read
    exactly that many elements on that device)."""
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")


def _same_device(like: torch.Tensor, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != like.device:
            raise ValueError(f"{name} is on {t.device}, expected {like.device}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def version() -> str:
    return load_library().h3attn_version().decode()


def frame_group_stride(grid, block_size: int = 64) -> int:
    """Query-block group stride for a T x H x W latent whose frames are whole blocks and that has
    at least four frames: H*W/64, so a sparse workgroup takes one spatial position in four
    consecutive frames. 1 otherwise (with fewer frames most of each four-block group would be
    empty)."""
    t, h, w = (int(x) for x in grid)
    frame = h * w
    if frame % block_size or t < 4:
        return 1
    return frame // block_size


def keep_count(n_blocks: int, sparsity: float) -> int:
    k = load_library().h3attn_keep_count(int(n_blocks), float(sparsity))
    if k < 0:
        raise ValueError(f"invalid n_blocks={n_blocks} or sparsity={sparsity}")
    return int(k)


def select_workspace_bytes(batch: int, heads: int, n_tokens: int, head_dim: int, block_size: int = 64) -> int:
    return int(load_library().h3attn_select_workspace_bytes(batch, heads, n_tokens, head_dim, block_size))


def _norm_rope_args(q, k, w_q, w_k, grid, sections, out, inplace):
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(w_q, "w_q", torch.float32, 1)
    _need(w_k, "w_k", torch.float32, 1)
    if q.shape != k.shape:
        raise ValueError("q and k must have the same shape")
    b, n, h, d = q.shape
    _need_shape(w_q, "w_q", (d,), q)
    _need_shape(w_k, "w_k", (d,), q)
    _same_device(q, k=k)
    if inplace:
        qo, ko = q, k
    elif out is not None:
        qo, ko = out
        _need(qo, "q_out", torch.bfloat16, 4)
        _need(ko, "k_out", torch.bfloat16, 4)
        _need_shape(qo, "q_out", q.shape, q)
        _need_shape(ko, "k_out", q.shape, q)
    else:
        qo, ko = torch.empty_like(q), torch.empty_like(k)
    g = Grid(*[int(x) for x in grid])
    if g.t * g.h * g.w != n:
        raise ValueError(f"grid {tuple(grid)} does not hold {n} tokens")
    d_t, d_h, d_w = [int(x) for x in sections]
    return qo, ko, g, (d_t, d_h, d_w)


def qk_norm_rope(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                 grid: Sequence[int], sections: Sequence[int], theta: float = 1e4, eps: float = 1e-6,
                 out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                 inplace: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fused per-head RMSNorm + 3D RoPE of bf16 q, k [B, N, heads, D]; returns (q', k')."""
    lib = load_library()
    qo, ko, g, (d_t, d_h, d_w) = _norm_rope_args(q, k, w_q, w_k, grid, sections, out, inplace)
    b, n, h, d = q.shape
    _check(lib.h3attn_qk_norm_rope(q.data_ptr(), k.data_ptr(), qo.data_ptr(), ko.data_ptr(),
                                   w_q.data_ptr(), w_k.data_ptr(), b, h, d, g, d_t, d_h, d_w,
                                   float(theta), float(eps), _stream()))
    return qo, ko


class PooledBlocks(NamedTuple):
    """The selection workspace as qk_norm_rope_pool left it, with the shape it was filled for."""
    workspace: torch.Tensor
    batch: int
    n_tokens: int
    heads: int
    head_dim: int
    block_size: int


def qk_norm_rope_pool(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                      grid: Sequence[int], sections: Sequence[int], theta: float = 1e4, eps: float = 1e-6,
                      block_size: int = 64, workspace: Optional[torch.Tensor] = None,
                      out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                      inplace: bool = False) -> Tuple[torch.Tensor, torch.Tensor, PooledBlocks]:
    """qk_norm_rope plus the selection's pooling of q', k' in the same pass; returns (q', k', pooled)
    for subblock_select_pooled."""
    lib = load_library()
    qo, ko, g, (d_t, d_h, d_w) = _norm_rope_args(q, k, w_q, w_k, grid, sections, out, inplace)
    b, n, h, d = q.shape
    need = select_workspace_bytes(b, h, n, d, block_size)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(q, workspace=workspace)
    _check(lib.h3attn_qk_norm_rope_pool(q.data_ptr(), k.data_ptr(), qo.data_ptr(), ko.data_ptr(),
                                        w_q.data_ptr(), w_k.data_ptr(), b, h, d, g, d_t, d_h, d_w,
                                        float(theta), float(eps), block_size, workspace.data_ptr(),
                                        workspace.numel(), _stream()))
    return qo, ko, PooledBlocks(workspace, b, n, h, d, block_size)


def subblock_select_pooled(pooled: PooledBlocks, sparsity: float, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """subblock_select on the q', k' of the qk_norm_rope_pool call that returned `pooled` (the same kept
    sets); int32 [B, heads, nB, keep], rows ascending. `pooled` serves one call (the selection rewrites
    the key blocks' exponents in the workspace in place)."""
    lib = load_library()
    ws = pooled.workspace
    _need(ws, "workspace", torch.uint8, 1)
    b, n, h, d, bs = pooled.batch, pooled.n_tokens, pooled.heads, pooled.head_dim, pooled.block_size
    nb = -(-n // bs)
    keep = keep_count(nb, sparsity)
    idx = torch.empty((b, h, nb, keep), dtype=torch.int32, device=ws.device) if out is None else out
    _need(idx, "block_idx", torch.int32, 4)
    _need_shape(idx, "block_idx", (b, h, nb, keep), ws)
    _check(lib.h3attn_subblock_select_pooled(b, h, n, d, bs, float(sparsity), keep, idx.data_ptr(), ws.data_ptr(),
                                             ws.numel(), _stream()))
    return idx


def dense_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, return_lse: bool = False,
              out: Optional[torch.Tensor] = None):
    """softmax(q k^T / sqrt(D)) v over the whole sequence, bf16 [B, N, heads, D]."""
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape")
    b, n, h, d = q.shape
    _same_device(q, k=k, v=v)
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", torch.bfloat16, 4)
    _need_shape(o, "out", q.shape, q)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.h3attn_dense_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _ptr(lse),
                                b, h, n, d, _stream()))
    return (o, lse) if return_lse else o


def subblock_select(q: torch.Tensor, k: torch.Tensor, sparsity: float, block_size: int = 64,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Kept key-block indices int32 [B, heads, nB, keep], rows ascending."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    if q.shape != k.shape:
        raise ValueError("q and k must have the same shape")
    b, n, h, d = q.shape
    nb = -(-n // block_size)
    keep = keep_count(nb, sparsity)
    need = select_workspace_bytes(b, h, n, d, block_size)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(q, k=k, workspace=workspace)
    idx = torch.empty((b, h, nb, keep), dtype=torch.int32, device=q.device) if out is None else out
    _need(idx, "block_idx", torch.int32, 4)
    _need_shape(idx, "block_idx", (b, h, nb, keep), q)
    _check(lib.h3attn_subblock_select(q.data_ptr(), k.data_ptr(), b, h, n, d, block_size, float(sparsity),
                                      keep, idx.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream()))
    return idx


def check_block_idx(block_idx: torch.Tensor) -> torch.Tensor:
    """Per-row validity flags of a kept set [B, heads, nB, keep] (uint8 [B, heads, nB]: 0 valid, bit 0
    an index outside [0, nB), bit 1 a repeated index), computed on the device."""
    lib = load_library()
    _need(block_idx, "block_idx", torch.int32, 4)
    b, h, nb, keep = block_idx.shape
    flags = torch.empty((b, h, nb), dtype=torch.uint8, device=block_idx.device)
    _check(lib.h3attn_check_block_idx(block_idx.data_ptr(), b, h, nb, keep, flags.data_ptr(), _stream()))
    return flags


def check_csr(row_ptr: torch.Tensor, col_idx: torch.Tensor, batch: int, heads: int, n_blocks: int) -> torch.Tensor:
    """Per-row validity flags of CSR kept sets (uint8 [B*heads*nB]: bits 0 and 1 as check_block_idx, bit 2
    a row whose range is decreasing or runs past col_idx)."""
    lib = load_library()
    _need(row_ptr, "row_ptr", torch.int64, 1)
    _need(col_idx, "col_idx", torch.int32, 1)
    rows = batch * heads * n_blocks
    if row_ptr.numel() != rows + 1:
        raise ValueError(f"row_ptr must have B*heads*nB + 1 = {rows + 1} entries")
    flags = torch.empty((rows,), dtype=torch.uint8, device=row_ptr.device)
    _check(lib.h3attn_check_csr(row_ptr.data_ptr(), _ptr(col_idx if col_idx.numel() > 0 else None), col_idx.numel(),
                                batch, heads, n_blocks, flags.data_ptr(), _stream()))
    return flags


def _raise_if_flagged(flags: torch.Tensor, what: str):
    bad = torch.nonzero(flags.reshape(-1)).reshape(-1)
    if bad.numel() > 0:
        r = int(bad[0])
        raise H3AttnError(1, f"{what}: {bad.numel()} invalid row(s), first row {r} (flags {int(flags.reshape(-1)[r])}: "
                             "1 out of range, 2 repeated index, 4 bad row range)")


def block_sparse_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_idx: torch.Tensor,
                     block_size: int = 64, return_lse: bool = False, out: Optional[torch.Tensor] = None,
                     group_stride: int = 1, validate: bool = False):
    """Attention of each 64-query block over its kept key blocks only. group_stride picks which
    four query blocks share a workgroup (i, i+S, i+2S, i+3S); it changes speed, never the result.
    validate=True first checks every kept-set row on the device (waits for the result) and raises
    H3AttnError on an index outside [0, nB) or a repeated one."""
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    _need(block_idx, "block_idx", torch.int32, 4)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape")
    b, n, h, d = q.shape
    nb = -(-n // block_size)
    if tuple(block_idx.shape[:3]) != (b, h, nb):
        raise ValueError(f"block_idx must be [B, heads, nB, keep] = [{b}, {h}, {nb}, keep]")
    keep = block_idx.shape[3]
    _same_device(q, k=k, v=v, block_idx=block_idx)
    if validate:
        _raise_if_flagged(check_block_idx(block_idx), "block_idx")
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", torch.bfloat16, 4)
    _need_shape(o, "out", q.shape, q)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device) if return_lse else None
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), block_idx.data_ptr(), keep, o.data_ptr(), _ptr(lse), b, h, n, d,
            block_size)
    if group_stride == 1:
        _check(lib.h3attn_block_sparse_fwd(*args, _stream()))
    else:
        _check(lib.h3attn_block_sparse_grouped_fwd(*args, group_stride, _stream()))
    return (o, lse) if return_lse else o


def threshold_workspace_bytes(batch: int, heads: int, n_tokens: int, head_dim: int, block_size: int = 64) -> int:
    return int(load_library().h3attn_threshold_workspace_bytes(batch, heads, n_tokens, head_dim, block_size))


def subblock_select_threshold(q: torch.Tensor, k: torch.Tensor, tau: float, block_size: int = 64,
                              workspace: Optional[torch.Tensor] = None):
    """Threshold-mode kept sets: every key block within tau of the row's best pooled score.
    Returns CSR (row_ptr int64 [B*heads*nB + 1], col_idx int32 [nnz]) over rows
    (b, head, query block). Waits for the count pass to read nnz before sizing col_idx."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    if q.shape != k.shape:
        raise ValueError("q and k must have the same shape")
    b, n, h, d = q.shape
    nb = -(-n // block_size)
    need = threshold_workspace_bytes(b, h, n, d, block_size)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(q, k=k, workspace=workspace)
    row_ptr = torch.empty((b * h * nb + 1,), dtype=torch.int64, device=q.device)
    st = _stream()
    _check(lib.h3attn_subblock_threshold_count(q.data_ptr(), k.data_ptr(), b, h, n, d, block_size, float(tau),
                                               row_ptr.data_ptr(), workspace.data_ptr(), workspace.numel(), st))
    nnz = int(row_ptr[-1].item())
    col_idx = torch.empty((max(nnz, 1),), dtype=torch.int32, device=q.device)
    _check(lib.h3attn_subblock_threshold_fill(b, h, n, d, block_size, row_ptr.data_ptr(), col_idx.data_ptr(), nnz,
                                              workspace.data_ptr(), workspace.numel(), st))
    return row_ptr, col_idx[:nnz]


def block_sparse_csr_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                         col_idx: torch.Tensor, block_size: int = 64, return_lse: bool = False,
                         out: Optional[torch.Tensor] = None, group_stride: int = 1, validate: bool = False):
    """Block-sparse attention with a variable kept set per query block (CSR rows). validate=True
    first checks every row on the device (as check_csr) and raises H3AttnError on a bad one."""
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    _need(row_ptr, "row_ptr", torch.int64, 1)
    _need(col_idx, "col_idx", torch.int32, 1)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape")
    b, n, h, d = q.shape
    nb = -(-n // block_size)
    if row_ptr.numel() != b * h * nb + 1:
        raise ValueError(f"row_ptr must have B*heads*nB + 1 = {b * h * nb + 1} entries")
    _same_device(q, k=k, v=v, row_ptr=row_ptr, col_idx=col_idx)
    if validate:
        _raise_if_flagged(check_csr(row_ptr, col_idx, b, h, nb), "CSR kept sets")
    o = torch.empty_like(q) if out is None else out
    _need(o, "out", torch.bfloat16, 4)
    _need_shape(o, "out", q.shape, q)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device) if return_lse else None
    ci = col_idx if col_idx.numel() > 0 else torch.zeros((1,), dtype=torch.int32, device=q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), row_ptr.data_ptr(), ci.data_ptr(), o.data_ptr(), _ptr(lse), b, h,
            n, d, block_size)
    if group_stride == 1:
        _check(lib.h3attn_block_sparse_csr_fwd(*args, _stream()))
    else:
        _check(lib.h3attn_block_sparse_csr_grouped_fwd(*args, group_stride, _stream()))
    return (o, lse) if return_lse else o


def adaln_modulate(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor, eps: float = 1e-6,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """LayerNorm(x) * (1 + scale) + shift over the hidden axis; x bf16 [B, N, C], shift/scale fp32 [B, C]."""
    lib = load_library()
    _need(x, "x", torch.bfloat16, 3)
    _need(shift, "shift", torch.float32, 2)
    _need(scale, "scale", torch.float32, 2)
    b, n, c = x.shape
    if tuple(shift.shape) != (b, c) or tuple(scale.shape) != (b, c):
        raise ValueError("shift and scale must be [B, C]")
    _same_device(x, shift=shift, scale=scale)
    o = torch.empty_like(x) if out is None else out
    _need(o, "out", torch.bfloat16, 3)
    _need_shape(o, "out", x.shape, x)
    _check(lib.h3attn_adaln_modulate(x.data_ptr(), shift.data_ptr(), scale.data_ptr(), o.data_ptr(), b, n, c,
                                     float(eps), _stream()))
    return o


def swiglu(gate: torch.Tensor, up: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """silu(gate) * up on bf16 tensors [..., F]. gate and up may be strided row views (e.g. the two
    halves of one [..., 2F] tensor) as long as the last axis is contiguous."""
    lib = load_library()
    for t, nm in ((gate, "gate"), (up, "up")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError(f"{nm} must be a bf16 device tensor")
        if t.stride(-1) != 1 or t.dim() < 1:
            raise ValueError(f"{nm} must have a contiguous last axis")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    f = gate.shape[-1]
    rows = gate.numel() // f
    def row_stride(t):
        if t.dim() == 1:
            return f
        t2 = t.reshape(-1, f) if t.is_contiguous() else t.view(-1, f)
        return t2.stride(0)
    _same_device(gate, up=up)
    o = torch.empty(gate.shape, dtype=torch.bfloat16, device=gate.device) if out is None else out
    _need(o, "out", torch.bfloat16)
    _need_shape(o, "out", gate.shape, gate)
    _check(lib.h3attn_swiglu(gate.data_ptr(), up.data_ptr(), o.data_ptr(), rows, f, row_stride(gate), row_stride(up),
                             _stream()))
    return o


def residual_change(cur: torch.Tensor, prev: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """float64 device tensor [2] = (sum |cur - prev|, sum |prev|) for two bf16 tensors."""
    lib = load_library()
    _need(cur, "cur", torch.bfloat16)
    _need(prev, "prev", torch.bfloat16)
    if cur.shape != prev.shape:
        raise ValueError("cur and prev must have the same shape")
    n = cur.numel()
    need = int(lib.h3attn_residual_workspace_bytes(n))
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=cur.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(cur, prev=prev, workspace=workspace)
    res = torch.empty((2,), dtype=torch.float64, device=cur.device) if out is None else out
    _need(res, "out", torch.float64, 1)
    _need_shape(res, "out", (2,), cur)
    _check(lib.h3attn_residual_change(cur.data_ptr(), prev.data_ptr(), n, res.data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), _stream()))
    return res


class CacheGate:
    """Cache-DiT reuse policy held in the library's C state (h3attn_cache_gate)."""

    CONSERVATIVE_MAX_CONSECUTIVE = 1
    STRIDE_MAX_CONSECUTIVE = 3

    def __init__(self, threshold: float, max_consecutive: int):
        self._lib = load_library()
        self._state = CacheGateState()
        _check(self._lib.h3attn_cache_gate_init(ctypes.byref(self._state), float(threshold), int(max_consecutive)))

    def decide(self, rel_change: float) -> bool:
        r = self._lib.h3attn_cache_gate_decide(ctypes.byref(self._state), float(rel_change))
        if r < 0:
            raise RuntimeError("invalid gate state")
        return bool(r)

    def step(self, cur: torch.Tensor, prev: Optional[torch.Tensor]) -> bool:
        """Measure the change of cur against prev on the GPU, read the two sums back and let the
        library form the ratio and decide (h3attn_cache_gate_decide_sums)."""
        sums = None
        if prev is not None:
            host = (ctypes.c_double * 2)(*residual_change(cur, prev).cpu().tolist())
            sums = ctypes.cast(host, ctypes.c_void_p)
        r = self._lib.h3attn_cache_gate_decide_sums(ctypes.byref(self._state), sums)
        if r < 0:
            raise RuntimeError("invalid gate state")
        return bool(r)


class Fp8QKV(NamedTuple):
    """e4m3 codes of q, k ([B, N, heads, D] uint8), of v transposed ([B, heads, D, nB*64] uint8,
    keys of each 64-key block in the order the P.V product reads them) and their power-of-two
    scales (float32 [B, heads, nB] for q and k, [B, heads, D] for v)."""
    q8: torch.Tensor
    k8: torch.Tensor
    v8t: torch.Tensor
    q_scale: torch.Tensor
    k_scale: torch.Tensor
    v_scale: torch.Tensor


def fp8_workspace_bytes(batch: int, heads: int, n_tokens: int, head_dim: int, block_size: int = 64) -> int:
    return int(load_library().h3attn_fp8_workspace_bytes(batch, heads, n_tokens, head_dim, block_size))


def fp8_quantize(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_size: int = 64,
                 workspace: Optional[torch.Tensor] = None, out: Optional[Fp8QKV] = None) -> Fp8QKV:
    """e4m3 quantisation of bf16 q, k (per 64-token block) and v (per channel) for the fp8 path."""
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must have the same shape")
    b, n, h, d = q.shape
    nb = -(-n // block_size)
    dev = q.device
    _same_device(q, k=k, v=v)
    if out is None:
        fq = Fp8QKV(torch.empty((b, n, h, d), dtype=torch.uint8, device=dev),
                    torch.empty((b, n, h, d), dtype=torch.uint8, device=dev),
                    torch.empty((b, h, d, nb * block_size), dtype=torch.uint8, device=dev),
                    torch.empty((b, h, nb), dtype=torch.float32, device=dev),
                    torch.empty((b, h, nb), dtype=torch.float32, device=dev),
                    torch.empty((b, h, d), dtype=torch.float32, device=dev))
    else:
        fq = out
        if _fp8_check(fq) != (b, n, h, d):
            raise ValueError("out tensors do not match q's shape")
        _same_device(q, q8=fq.q8, k8=fq.k8, v8t=fq.v8t, q_scale=fq.q_scale, k_scale=fq.k_scale, v_scale=fq.v_scale)
    need = fp8_workspace_bytes(b, h, n, d, block_size)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _same_device(q, workspace=workspace)
    _check(lib.h3attn_fp8_quantize(q.data_ptr(), k.data_ptr(), v.data_ptr(), fq.q8.data_ptr(), fq.k8.data_ptr(),
                                   fq.v8t.data_ptr(), fq.q_scale.data_ptr(), fq.k_scale.data_ptr(),
                                   fq.v_scale.data_ptr(), b, h, n, d, block_size, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream()))
    return fq


def _fp8_check(fq: Fp8QKV):
    for t, nm in ((fq.q8, "q8"), (fq.k8, "k8"), (fq.v8t, "v8t")):
        _need(t, nm, torch.uint8, 4)
    for t, nm in ((fq.q_scale, "q_scale"), (fq.k_scale, "k_scale"), (fq.v_scale, "v_scale")):
        _need(t, nm, torch.float32, 3)
    b, n, h, d = fq.q8.shape
    nb = -(-n // 64)
    if fq.k8.shape != fq.q8.shape or tuple(fq.v8t.shape) != (b, h, d, nb * 64) or \
            tuple(fq.q_scale.shape) != (b, h, nb) or tuple(fq.k_scale.shape) != (b, h, nb) or \
            tuple(fq.v_scale.shape) != (b, h, d):
        raise ValueError("inconsistent fp8 tensors")
    _same_device(fq.q8, k8=fq.k8, v8t=fq.v8t, q_scale=fq.q_scale, k_scale=fq.k_scale, v_scale=fq.v_scale)
    return b, n, h, d


def fp8_dense_fwd(fq: Fp8QKV, return_lse: bool = False, out: Optional[torch.Tensor] = None):
    """Dense attention on e4m3 tensors from fp8_quantize; bf16 output [B, N, heads, D]."""
    lib = load_library()
    b, n, h, d = _fp8_check(fq)
    o = torch.empty((b, n, h, d), dtype=torch.bfloat16, device=fq.q8.device) if out is None else out
    _need(o, "out", torch.bfloat16, 4)
    _need_shape(o, "out", (b, n, h, d), fq.q8)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=o.device) if return_lse else None
    _check(lib.h3attn_fp8_dense_fwd(fq.q8.data_ptr(), fq.k8.data_ptr(), fq.v8t.data_ptr(), fq.q_scale.data_ptr(),
                                    fq.k_scale.data_ptr(), fq.v_scale.data_ptr(), o.data_ptr(), _ptr(lse), b, h, n, d,
                                    64, _stream()))
    return (o, lse) if return_lse else o


def fp8_block_sparse_fwd(fq: Fp8QKV, block_idx: torch.Tensor, return_lse: bool = False,
                         out: Optional[torch.Tensor] = None, group_stride: int = 1, validate: bool = False):
    """Block-sparse attention on e4m3 tensors over the kept key blocks block_idx [B, heads, nB, keep]
    (validate as in block_sparse_fwd)."""
    lib = load_library()
    b, n, h, d = _fp8_check(fq)
    _need(block_idx, "block_idx", torch.int32, 4)
    nb = -(-n // 64)
    if tuple(block_idx.shape[:3]) != (b, h, nb):
        raise ValueError(f"block_idx must be [B, heads, nB, keep] = [{b}, {h}, {nb}, keep]")
    keep = block_idx.shape[3]
    _same_device(fq.q8, block_idx=block_idx)
    if validate:
        _raise_if_flagged(check_block_idx(block_idx), "block_idx")
    o = torch.empty((b, n, h, d), dtype=torch.bfloat16, device=fq.q8.device) if out is None else out
    _need(o, "out", torch.bfloat16, 4)
    _need_shape(o, "out", (b, n, h, d), fq.q8)
    lse = torch.empty((b, h, n), dtype=torch.float32, device=o.device) if return_lse else None
    _check(lib.h3attn_fp8_block_sparse_fwd(fq.q8.data_ptr(), fq.k8.data_ptr(), fq.v8t.data_ptr(),
                                           fq.q_scale.data_ptr(), fq.k_scale.data_ptr(), fq.v_scale.data_ptr(),
                                           block_idx.data_ptr(), keep, o.data_ptr(), _ptr(lse), b, h, n, d, 64,
                                           group_stride, _stream()))
    return (o, lse) if return_lse else o
