"""MSA (MiniMax Sparse Attention) layer hot path on MI355X (gfx950).

Thin Python binding of the C ABI in include/msa.h (libmsa.so, hand-written HIP
kernels). This module only marshals arguments: it checks tensor shapes, sizes
the workspace, allocates outputs with torch and passes raw device pointers and
the current HIP stream. Every step of the path runs in the library's kernels;
there is no fallback. If libmsa.so is missing the calls raise.

Functions (same names as the C entry points):
  msa_select(q_idx, k_idx, topk, q_start=0, ...)     -> block ids (+ scores, margin)
  msa_attn_fwd(q, k, v, block_ids, q_start=0, ...)   -> (out, lse)
  msa_attn_fwd_noalloc(q, k, v, block_ids, out, lse, ...)
                                                     -> the same, on a fixed device scratch
  msa_kl_align(q, k, q_idx, k_idx, block_ids, lse_main, q_start=0, ...)
                                                     -> kl_rows, kl_mean, dlogits
  msa_attn_bwd(q, k, v, block_ids, out, lse, dout, q_start=0, ...)
                                                     -> (dq, dk, dv)
  msa_idx_bwd(q_idx, k_idx, block_ids, dlogits, coef, q_start=0, ...)
                                                     -> (dq_idx, dk_idx)
  msa_dense_lse(q, k, q_start=0, ...)                -> lse_main over the full causal context
  msa_kl_dense(q, k, q_idx, k_idx, lse_main, q_start=0, ...)
                                                     -> kl_rows, kl_mean, lse_idx, block_mass
  msa_kl_dense_bwd(q, k, q_idx, k_idx, lse_main, coef, q_start=0, ...)
                                                     -> the same + dq_idx, dk_idx
  msa_block_recall(block_mass, block_ids, q_start=0, ...)
                                                     -> block_recall, score_recall, means
  msa_index_quantize_fp8(q_idx, k_idx, ...)          -> q8, q_exp, k8, k_exp (OCP E4M3)
  msa_select_fp8(q8, q_exp, k8, k_exp, topk, ...)    -> block ids (+ scores, margin)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (loads the HIP runtime that libmsa.so binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")
# the same kernel and API objects linked with the kernel-timing hook (include/msa_timing.h)
TIMED_LIB_PATH = os.path.join(_HERE, "libmsa_timed.so")

(MSA_OK, MSA_ERR_NULL, MSA_ERR_SHAPE, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_DEVICE,
 MSA_ERR_SCRATCH) = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20  # fixed device scratch of msa_attn_fwd_noalloc
MSA_F32, MSA_BF16 = 0, 1
MSA_OP_SELECT, MSA_OP_ATTN, MSA_OP_KL, MSA_OP_ATTN_BWD, MSA_OP_IDX_BWD = 0, 1, 2, 3, 4
MSA_OP_KL_DENSE_BWD = 5
KERNELS = ["index_blockmax", "topk", "bucket_hist", "bucket_scan", "bucket_scatter",
           "work_items", "sparse_attn", "combine", "kl_idx_stats", "kl_idx_lse", "kl_main",
           "kl_reduce", "attn_bwd", "idx_bwd", "dense_lse", "kl_dense", "recall", "dense_lse_idx", "index_fp8", "quantize_fp8", "kl_dense_chain",
           "bucket_sort", "bwd_finalize"]
EXPORTS = ["msa_workspace_size", "msa_select", "msa_attn_fwd", "msa_kl_align", "msa_attn_bwd",
           "msa_idx_bwd", "msa_dense_lse", "msa_kl_dense", "msa_kl_dense_bwd", "msa_block_recall",
           "msa_index_quantize_fp8", "msa_select_fp8", "msa_status_string",
           "msa_attn_fwd_noalloc", "msa_index_block_lse"]
TIMING_EXPORTS = ["msa_prof_begin", "msa_prof_end"]


class MsaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seqlen_kv", "seqlen_q", "q_start", "num_q_heads", "num_kv_heads", "head_dim",
        "idx_dim", "block_size", "topk", "dtype")]


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None
_timed = False


def use_timed_build() -> None:
    """Route every call through libmsa_timed.so, the measurement build whose launches can be
    timed with KernelTimer. Must be called before the first call into the library."""
    global _timed
    if _lib is not None and not _timed:
        raise RuntimeError("the product library is already loaded")
    _timed = True


def lib() -> ctypes.CDLL:
    """The loaded libmsa.so (libmsa_timed.so after use_timed_build()); raises if it has not
    been built."""
    global _lib
    if _lib is None:
        path = TIMED_LIB_PATH if _timed else LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python learned_kv_block_amd/build.py` (or __graft_entry__.build())")
        L = ctypes.CDLL(path)
        P, S = ctypes.c_void_p, ctypes.POINTER(MsaShape)
        L.msa_workspace_size.argtypes = [S, ctypes.c_int]
        L.msa_workspace_size.restype = ctypes.c_size_t
        L.msa_select.argtypes = [S, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_attn_fwd.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_attn_fwd_noalloc.argtypes = [S, P, P, P, P, P, P, P]
        L.msa_kl_align.argtypes = [S, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_attn_bwd.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_idx_bwd.argtypes = [S, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
        L.msa_dense_lse.argtypes = [S, P, P, P, P]
        L.msa_kl_dense.argtypes = [S, P, P, P, P, P, P, P, P, P, P]
        L.msa_block_recall.argtypes = [S, P, P, P, P, P, P]
        L.msa_kl_dense_bwd.argtypes = [S, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P,
                                       ctypes.c_size_t, P]
        L.msa_index_quantize_fp8.argtypes = [S, P, P, P, P, P, P, P]
        L.msa_select_fp8.argtypes = [S, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.msa_index_block_lse.argtypes = [S, P, P, P, P, P]
        for f in ("msa_select", "msa_index_block_lse", "msa_attn_fwd", "msa_attn_fwd_noalloc",
                  "msa_kl_align",
                  "msa_attn_bwd", "msa_idx_bwd",
                  "msa_dense_lse", "msa_kl_dense", "msa_kl_dense_bwd", "msa_block_recall",
                  "msa_index_quantize_fp8", "msa_select_fp8"):
            getattr(L, f).restype = ctypes.c_int
        L.msa_status_string.argtypes = [ctypes.c_int]
        L.msa_status_string.restype = ctypes.c_char_p
        if _timed:
            L.msa_prof_begin.argtypes = [ctypes.c_int, ctypes.c_int]
            L.msa_prof_end.argtypes = [ctypes.POINTER(ctypes.c_float),
                                       ctypes.POINTER(ctypes.c_int)]
            L.msa_prof_begin.restype = ctypes.c_int
            L.msa_prof_end.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().msa_status_string(int(status)).decode()


def make_shape(batch, seqlen_kv, seqlen_q, q_start, num_q_heads, num_kv_heads, head_dim,
               idx_dim, topk, dtype, block_size=128) -> MsaShape:
    return MsaShape(batch, seqlen_kv, seqlen_q, q_start, num_q_heads, num_kv_heads, head_dim,
                    idx_dim, block_size, topk, dtype)


def workspace_size(shape: MsaShape, op: int) -> int:
    return int(lib().msa_workspace_size(ctypes.byref(shape), op))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    if t.dtype == torch.float32:
        return MSA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor, got {tuple(t.shape)}")


def _expect(t: torch.Tensor, name: str, shape, dtype=None):
    """t must be a contiguous tensor of `shape` (None leaves a dimension free) and, when given,
    of `dtype`. The library sees raw pointers only, so every size it derives from the shape
    descriptor must match the buffers it is handed."""
    _check(t, name, len(shape))
    for ax, (got, want) in enumerate(zip(t.shape, shape)):
        if want is not None and got != want:
            raise ValueError(f"{name} has shape {tuple(t.shape)}; dimension {ax} must be {want}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _on_device(*tensors):
    """Every tensor must live on the same GPU (checked after the shapes and dtypes)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(shape: MsaShape, op: int, device, workspace: Optional[torch.Tensor]):
    n = workspace_size(shape, op)
    if n == 0:
        return None, 0
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != torch.device(device):
            raise ValueError(f"workspace must be a device tensor on {device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.numel() * workspace.element_size() < n:
            raise ValueError(f"workspace of {workspace.numel()} bytes < {n} required")
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(n, dtype=torch.uint8, device=device), n


def shape_for(q_idx: torch.Tensor, k_idx: torch.Tensor, topk: int, q_start: int = 0,
              num_q_heads: Optional[int] = None, head_dim: int = 128) -> MsaShape:
    B, Nq, Hkv, DI = q_idx.shape
    N = k_idx.shape[1]
    Hq = num_q_heads if num_q_heads is not None else Hkv
    return make_shape(B, N, Nq, q_start, Hq, Hkv, head_dim, DI, topk, _dtype_code(q_idx))


def msa_select(q_idx: torch.Tensor, k_idx: torch.Tensor, topk: int, q_start: int = 0,
               want_scores: bool = False, want_margin: bool = False,
               num_q_heads: Optional[int] = None, head_dim: int = 128,
               workspace: Optional[torch.Tensor] = None):
    """Block selection. q_idx [B, Nq, Hkv, d_idx], k_idx [B, N, d_idx] (bf16/fp32, device).

    Returns dict(ids [B, Nq, Hkv, topk] int32, block_scores [B, Nq, Hkv, nb] fp32 (opt),
    margin [B, Nq, Hkv] fp32 (opt)). num_q_heads / head_dim only enter the shape check."""
    _check(q_idx, "q_idx", 4)
    B, Nq, Hkv, DI = q_idx.shape
    _expect(k_idx, "k_idx", (B, None, DI), q_idx.dtype)
    _on_device(q_idx, k_idx)
    sh = shape_for(q_idx, k_idx, topk, q_start, num_q_heads, head_dim)
    nb = (k_idx.shape[1] + 127) // 128
    dev = q_idx.device
    ids = torch.empty((B, Nq, Hkv, topk), dtype=torch.int32, device=dev)
    scores = torch.empty((B, Nq, Hkv, nb), dtype=torch.float32, device=dev) if want_scores else None
    margin = torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev) if want_margin else None
    ws, nws = (None, 0) if want_scores else _workspace(sh, MSA_OP_SELECT, dev, workspace)
    st = lib().msa_select(ctypes.byref(sh), _ptr(q_idx), _ptr(k_idx), _ptr(ids), _ptr(scores),
                          _ptr(margin), _ptr(ws), nws, _stream(q_idx))
    if st != MSA_OK:
        raise MsaError(st, "msa_select")
    out = {"ids": ids}
    if want_scores:
        out["block_scores"] = scores
    if want_margin:
        out["margin"] = margin
    return out


def msa_index_block_lse(q_idx: torch.Tensor, k_idx: torch.Tensor, q_start: int = 0,
                        num_q_heads: Optional[int] = None, head_dim: int = 128):
    """Index forward with per-block LSE. q_idx [B, Nq, Hkv, d_idx], k_idx [B, N, d_idx].

    Returns dict(block_scores, block_lse), both [B, Nq, Hkv, nb] fp32, -inf past each row's
    local block. num_q_heads / head_dim only enter the shape check."""
    _check(q_idx, "q_idx", 4)
    B, Nq, Hkv, DI = q_idx.shape
    _expect(k_idx, "k_idx", (B, None, DI), q_idx.dtype)
    _on_device(q_idx, k_idx)
    sh = shape_for(q_idx, k_idx, 1, q_start, num_q_heads, head_dim)
    nb = (k_idx.shape[1] + 127) // 128
    dev = q_idx.device
    scores = torch.empty((B, Nq, Hkv, nb), dtype=torch.float32, device=dev)
    blse = torch.empty((B, Nq, Hkv, nb), dtype=torch.float32, device=dev)
    st = lib().msa_index_block_lse(ctypes.byref(sh), _ptr(q_idx), _ptr(k_idx), _ptr(scores),
                                   _ptr(blse), _stream(q_idx))
    if st != MSA_OK:
        raise MsaError(st, "msa_index_block_lse")
    return {"block_scores": scores, "block_lse": blse}


def msa_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_ids: torch.Tensor,
                 q_start: int = 0, idx_dim: int = 64, workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Sparse attention over the selected blocks. q [B, Nq, Hq, d], k/v [B, N, Hkv, d],
    block_ids [B, Nq, Hkv, topk]. Returns (out [B, Nq, Hq, d], lse [B, Nq, Hq] fp32)."""
    _check(q, "q", 4)
    B, Nq, Hq, D = q.shape
    _expect(k, "k", (B, None, None, D), q.dtype)
    N, Hkv = k.shape[1], k.shape[2]
    _expect(v, "v", tuple(k.shape), q.dtype)
    _expect(block_ids, "block_ids", (B, Nq, Hkv, None), torch.int32)
    if out is not None:
        _expect(out, "out", tuple(q.shape), q.dtype)
    if lse is not None:
        _expect(lse, "lse", (B, Nq, Hq), torch.float32)
    _on_device(q, k, v, block_ids, out, lse)
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, D, idx_dim, block_ids.shape[3], _dtype_code(q))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    ws, nws = _workspace(sh, MSA_OP_ATTN, q.device, workspace)
    st = lib().msa_attn_fwd(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(block_ids),
                            _ptr(out), _ptr(lse), _ptr(ws), nws, _stream(q))
    if st != MSA_OK:
        raise MsaError(st, "msa_attn_fwd")
    return out, lse


def msa_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         block_ids: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                         q_start: int = 0, idx_dim: int = 64):
    """msa_attn_fwd without a workspace: the library's fixed 64 MiB device scratch is used
    (for callers that cannot allocate). The caller passes the outputs; calls that overlap
    on one GPU race on the scratch. Raises MsaError(MSA_ERR_SCRATCH) for larger workloads."""
    _check(q, "q", 4)
    B, Nq, Hq, D = q.shape
    _expect(k, "k", (B, None, None, D), q.dtype)
    N, Hkv = k.shape[1], k.shape[2]
    _expect(v, "v", tuple(k.shape), q.dtype)
    _expect(block_ids, "block_ids", (B, Nq, Hkv, None), torch.int32)
    _expect(out, "out", tuple(q.shape), q.dtype)
    _expect(lse, "lse", (B, Nq, Hq), torch.float32)
    _on_device(q, k, v, block_ids, out, lse)
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, D, idx_dim, block_ids.shape[3], _dtype_code(q))
    st = lib().msa_attn_fwd_noalloc(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(block_ids),
                                    _ptr(out), _ptr(lse), _stream(q))
    if st != MSA_OK:
        raise MsaError(st, "msa_attn_fwd_noalloc")
    return out, lse


def msa_kl_align(q: torch.Tensor, k: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor,
                 block_ids: torch.Tensor, lse_main: torch.Tensor, q_start: int = 0,
                 want_dlogits: bool = True, workspace: Optional[torch.Tensor] = None):
    """KL alignment on the selected support. Returns dict(kl_rows [B, Nq, Hkv],
    kl_mean [1], dlogits [B, Nq, Hkv, topk, 128] (opt)), all fp32."""
    _check(q, "q", 4)
    B, Nq, Hq, D = q.shape
    _expect(k, "k", (B, None, None, D), q.dtype)
    N, Hkv = k.shape[1], k.shape[2]
    _expect(q_idx, "q_idx", (B, Nq, Hkv, None), q.dtype)
    _expect(k_idx, "k_idx", (B, N, q_idx.shape[3]), q.dtype)
    _expect(block_ids, "block_ids", (B, Nq, Hkv, None), torch.int32)
    _expect(lse_main, "lse_main", (B, Nq, Hq), torch.float32)
    _on_device(q, k, q_idx, k_idx, block_ids, lse_main)
    K = block_ids.shape[3]
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, D, q_idx.shape[3], K, _dtype_code(q))
    dev = q.device
    kl_rows = torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev)
    kl_mean = torch.empty((1,), dtype=torch.float32, device=dev)
    dl = torch.empty((B, Nq, Hkv, K, 128), dtype=torch.float32, device=dev) if want_dlogits else None
    ws, nws = _workspace(sh, MSA_OP_KL, dev, workspace)
    st = lib().msa_kl_align(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx),
                            _ptr(block_ids), _ptr(lse_main), _ptr(kl_rows), _ptr(kl_mean),
                            _ptr(dl), _ptr(ws), nws, _stream(q))
    if st != MSA_OK:
        raise MsaError(st, "msa_kl_align")
    out = {"kl_rows": kl_rows, "kl_mean": kl_mean}
    if want_dlogits:
        out["dlogits"] = dl
    return out


def msa_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_ids: torch.Tensor,
                 out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor, q_start: int = 0,
                 idx_dim: int = 64, workspace: Optional[torch.Tensor] = None):
    """Gradients of msa_attn_fwd with the selection fixed: (dq like q, dk like k, dv like v)."""
    _check(q, "q", 4)
    B, Nq, Hq, D = q.shape
    _expect(k, "k", (B, None, None, D), q.dtype)
    N, Hkv = k.shape[1], k.shape[2]
    _expect(v, "v", tuple(k.shape), q.dtype)
    _expect(block_ids, "block_ids", (B, Nq, Hkv, None), torch.int32)
    _expect(out, "out", tuple(q.shape), q.dtype)
    _expect(dout, "dout", tuple(q.shape), q.dtype)
    _expect(lse, "lse", (B, Nq, Hq), torch.float32)
    _on_device(q, k, v, block_ids, out, dout, lse)
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, D, idx_dim, block_ids.shape[3], _dtype_code(q))
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws, nws = _workspace(sh, MSA_OP_ATTN_BWD, q.device, workspace)
    st = lib().msa_attn_bwd(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(block_ids),
                            _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                            _ptr(ws), nws, _stream(q))
    if st != MSA_OK:
        raise MsaError(st, "msa_attn_bwd")
    return dq, dk, dv


def msa_idx_bwd(q_idx: torch.Tensor, k_idx: torch.Tensor, block_ids: torch.Tensor,
                dlogits: torch.Tensor, coef: float = 1.0, q_start: int = 0, num_q_heads: int = 64,
                head_dim: int = 128, workspace: Optional[torch.Tensor] = None):
    """Index-logit gradient chained into the index projections: (dq_idx like q_idx,
    dk_idx like k_idx). dlogits [B, Nq, Hkv, topk, 128] fp32 as msa_kl_align returns it."""
    _check(q_idx, "q_idx", 4)
    B, Nq, Hkv, DI = q_idx.shape
    _expect(k_idx, "k_idx", (B, None, DI), q_idx.dtype)
    _expect(block_ids, "block_ids", (B, Nq, Hkv, None), torch.int32)
    _expect(dlogits, "dlogits", (B, Nq, Hkv, block_ids.shape[3], 128), torch.float32)
    _on_device(q_idx, k_idx, block_ids, dlogits)
    sh = shape_for(q_idx, k_idx, block_ids.shape[3], q_start, num_q_heads, head_dim)
    dq = torch.empty_like(q_idx)
    dk = torch.empty_like(k_idx)
    ws, nws = _workspace(sh, MSA_OP_IDX_BWD, q_idx.device, workspace)
    st = lib().msa_idx_bwd(ctypes.byref(sh), _ptr(q_idx), _ptr(k_idx), _ptr(block_ids),
                           _ptr(dlogits), float(coef), _ptr(dq), _ptr(dk), _ptr(ws), nws,
                           _stream(q_idx))
    if st != MSA_OK:
        raise MsaError(st, "msa_idx_bwd")
    return dq, dk


def msa_dense_lse(q: torch.Tensor, k: torch.Tensor, q_start: int = 0, idx_dim: int = 64):
    """LSE of the main branch over the full causal context: fp32 [B, Nq, Hq]."""
    _check(q, "q", 4)
    B, Nq, Hq, D = q.shape
    _expect(k, "k", (B, None, None, D), q.dtype)
    _on_device(q, k)
    N, Hkv = k.shape[1], k.shape[2]
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, D, idx_dim, 1, _dtype_code(q))
    lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    st = lib().msa_dense_lse(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(lse), _stream(q))
    if st != MSA_OK:
        raise MsaError(st, "msa_dense_lse")
    return lse


def msa_kl_dense(q: torch.Tensor, k: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor,
                 lse_main: torch.Tensor, q_start: int = 0, want_mass: bool = True):
    """KL alignment on the full causal context (warm-up stage): dict(kl_rows [B, Nq, Hkv],
    kl_mean [1], lse_idx [B, Nq, Hkv], block_mass [B, Nq, Hkv, nb] (opt)), all fp32."""
    _check(q, "q", 4)
    B, Nq, Hq, D = q.shape
    _expect(k, "k", (B, None, None, D), q.dtype)
    N, Hkv = k.shape[1], k.shape[2]
    _expect(q_idx, "q_idx", (B, Nq, Hkv, None), q.dtype)
    _expect(k_idx, "k_idx", (B, N, q_idx.shape[3]), q.dtype)
    _expect(lse_main, "lse_main", (B, Nq, Hq), torch.float32)
    _on_device(q, k, q_idx, k_idx, lse_main)
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, D, q_idx.shape[3], 1, _dtype_code(q))
    dev = q.device
    nb = (N + 127) // 128
    kl_rows = torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev)
    kl_mean = torch.empty((1,), dtype=torch.float32, device=dev)
    lse_idx = torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev)
    mass = torch.empty((B, Nq, Hkv, nb), dtype=torch.float32, device=dev) if want_mass else None
    st = lib().msa_kl_dense(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx),
                            _ptr(lse_main), _ptr(lse_idx), _ptr(kl_rows), _ptr(kl_mean),
                            _ptr(mass), _stream(q))
    if st != MSA_OK:
        raise MsaError(st, "msa_kl_dense")
    out = {"kl_rows": kl_rows, "kl_mean": kl_mean, "lse_idx": lse_idx}
    if want_mass:
        out["block_mass"] = mass
    return out


def msa_kl_dense_bwd(q: torch.Tensor, k: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor,
                     lse_main: torch.Tensor, coef: float = 1.0, q_start: int = 0,
                     want_kl: bool = True, want_mass: bool = False,
                     workspace: Optional[torch.Tensor] = None):
    """The full-context KL with its gradient into the index projections: dict(dq_idx like
    q_idx, dk_idx like k_idx, lse_idx, and kl_rows / kl_mean / block_mass when asked)."""
    _check(q, "q", 4)
    B, Nq, Hq, D = q.shape
    _expect(k, "k", (B, None, None, D), q.dtype)
    N, Hkv = k.shape[1], k.shape[2]
    _expect(q_idx, "q_idx", (B, Nq, Hkv, None), q.dtype)
    _expect(k_idx, "k_idx", (B, N, q_idx.shape[3]), q.dtype)
    _expect(lse_main, "lse_main", (B, Nq, Hq), torch.float32)
    _on_device(q, k, q_idx, k_idx, lse_main)
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, D, q_idx.shape[3], 1, _dtype_code(q))
    dev = q.device
    nb = (N + 127) // 128
    out = {"lse_idx": torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev),
           "dq_idx": torch.empty_like(q_idx), "dk_idx": torch.empty_like(k_idx)}
    if want_kl:
        out["kl_rows"] = torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev)
        out["kl_mean"] = torch.empty((1,), dtype=torch.float32, device=dev)
    if want_mass:
        out["block_mass"] = torch.empty((B, Nq, Hkv, nb), dtype=torch.float32, device=dev)
    ws, nws = _workspace(sh, MSA_OP_KL_DENSE_BWD, dev, workspace)
    st = lib().msa_kl_dense_bwd(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx),
                                _ptr(lse_main), float(coef), _ptr(out["lse_idx"]),
                                _ptr(out.get("kl_rows")), _ptr(out.get("kl_mean")),
                                _ptr(out.get("block_mass")), _ptr(out["dq_idx"]),
                                _ptr(out["dk_idx"]), _ptr(ws), nws, _stream(q))
    if st != MSA_OK:
        raise MsaError(st, "msa_kl_dense_bwd")
    return out


def msa_block_recall(block_mass: torch.Tensor, block_ids: torch.Tensor, q_start: int = 0,
                     seqlen_kv: Optional[int] = None, num_q_heads: Optional[int] = None,
                     head_dim: int = 128, idx_dim: int = 64):
    """Block recall and score recall of block_ids [B, Nq, Hkv, topk] against the teacher's
    block masses [B, Nq, Hkv, nb]: dict(block_recall, score_recall [B, Nq, Hkv], means [2])."""
    _expect(block_mass, "block_mass", (None, None, None, None), torch.float32)
    B, Nq, Hkv, nb = block_mass.shape
    _expect(block_ids, "block_ids", (B, Nq, Hkv, None), torch.int32)
    _on_device(block_mass, block_ids)
    N = seqlen_kv if seqlen_kv is not None else nb * 128
    if (N + 127) // 128 != nb:
        raise ValueError("seqlen_kv does not match the block count of block_mass")
    Hq = num_q_heads if num_q_heads is not None else Hkv
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, head_dim, idx_dim, block_ids.shape[3], MSA_BF16)
    dev = block_mass.device
    brec = torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev)
    srec = torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev)
    means = torch.empty((2,), dtype=torch.float32, device=dev)
    st = lib().msa_block_recall(ctypes.byref(sh), _ptr(block_mass), _ptr(block_ids), _ptr(brec),
                                _ptr(srec), _ptr(means), _stream(block_mass))
    if st != MSA_OK:
        raise MsaError(st, "msa_block_recall")
    return {"block_recall": brec, "score_recall": srec, "means": means}


def msa_index_quantize_fp8(q_idx: Optional[torch.Tensor], k_idx: Optional[torch.Tensor],
                           seqlen_kv: Optional[int] = None, q_start: int = 0,
                           num_q_heads: Optional[int] = None, head_dim: int = 128):
    """OCP E4M3 index inputs with power-of-two scales per Q_idx row / K_idx block:
    dict(q8 uint8 [B, Nq, Hkv, d_idx], q_exp int32 [B, Nq, Hkv]) for q_idx and/or
    dict(k8 uint8 [B, N, d_idx], k_exp int32 [B, nb]) for k_idx (either may be None)."""
    if q_idx is None and k_idx is None:
        raise ValueError("nothing to quantize")
    ref = q_idx if q_idx is not None else k_idx
    if q_idx is not None:
        _check(q_idx, "q_idx", 4)
        B, Nq, Hkv, DI = q_idx.shape
    if k_idx is not None:
        if q_idx is not None:
            _expect(k_idx, "k_idx", (B, None, DI), q_idx.dtype)
        _check(k_idx, "k_idx", 3)
        B, N, DI = k_idx.shape
    else:
        N = seqlen_kv if seqlen_kv is not None else q_start + Nq
    _on_device(q_idx, k_idx)
    if q_idx is None:
        Nq, Hkv = 1, 1
        q_start = N - 1
    Hq = num_q_heads if num_q_heads is not None else Hkv
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, head_dim, DI, 1, _dtype_code(ref))
    dev = ref.device
    out = {}
    q8 = qe = k8 = ke = None
    if q_idx is not None:
        q8 = torch.empty(q_idx.shape, dtype=torch.uint8, device=dev)
        qe = torch.empty(q_idx.shape[:3], dtype=torch.int32, device=dev)
        out.update(q8=q8, q_exp=qe)
    if k_idx is not None:
        k8 = torch.empty(k_idx.shape, dtype=torch.uint8, device=dev)
        ke = torch.empty((B, (N + 127) // 128), dtype=torch.int32, device=dev)
        out.update(k8=k8, k_exp=ke)
    st = lib().msa_index_quantize_fp8(ctypes.byref(sh), _ptr(q_idx), _ptr(k_idx), _ptr(q8),
                                      _ptr(qe), _ptr(k8), _ptr(ke), _stream(ref))
    if st != MSA_OK:
        raise MsaError(st, "msa_index_quantize_fp8")
    return out


def msa_select_fp8(q8: torch.Tensor, q_exp: torch.Tensor, k8: torch.Tensor, k_exp: torch.Tensor,
                   topk: int, q_start: int = 0, want_scores: bool = False,
                   want_margin: bool = False, num_q_heads: Optional[int] = None,
                   head_dim: int = 128, workspace: Optional[torch.Tensor] = None):
    """msa_select on FP8 index inputs (as msa_index_quantize_fp8 returns them)."""
    _expect(q8, "q8", (None, None, None, None), torch.uint8)
    B, Nq, Hkv, DI = q8.shape
    _expect(k8, "k8", (B, None, DI), torch.uint8)
    N = k8.shape[1]
    _expect(q_exp, "q_exp", (B, Nq, Hkv), torch.int32)
    _expect(k_exp, "k_exp", (B, (N + 127) // 128), torch.int32)
    _on_device(q8, k8, q_exp, k_exp)
    Hq = num_q_heads if num_q_heads is not None else Hkv
    sh = make_shape(B, N, Nq, q_start, Hq, Hkv, head_dim, DI, topk, MSA_BF16)
    nb = (N + 127) // 128
    dev = q8.device
    ids = torch.empty((B, Nq, Hkv, topk), dtype=torch.int32, device=dev)
    scores = torch.empty((B, Nq, Hkv, nb), dtype=torch.float32, device=dev) if want_scores else None
    margin = torch.empty((B, Nq, Hkv), dtype=torch.float32, device=dev) if want_margin else None
    ws, nws = (None, 0) if want_scores else _workspace(sh, MSA_OP_SELECT, dev, workspace)
    st = lib().msa_select_fp8(ctypes.byref(sh), _ptr(q8), _ptr(q_exp), _ptr(k8), _ptr(k_exp),
                              _ptr(ids), _ptr(scores), _ptr(margin), _ptr(ws), nws, _stream(q8))
    if st != MSA_OK:
        raise MsaError(st, "msa_select_fp8")
    out = {"ids": ids}
    if want_scores:
        out["block_scores"] = scores
    if want_margin:
        out["margin"] = margin
    return out


class KernelTimer:
    """Durations of kernel launches, from HIP events the library records on the launch
    stream: one kernel (by name) or every kernel (kernel=None). Needs the measurement build:
    call use_timed_build() first.

    After the block: total_ms / launches for the named kernel (or all kernels), and
    per_kernel = {name: (total_ms, launches)} for every kernel that ran."""

    def __init__(self, kernel: Optional[str] = None, max_launches: int = 1000):
        if not _timed:
            raise RuntimeError("KernelTimer needs the measurement build (use_timed_build())")
        self.kid = -1 if kernel is None else KERNELS.index(kernel)
        self.max = max_launches
        self.total_ms = 0.0
        self.launches = 0
        self.per_kernel = {}

    def __enter__(self):
        st = lib().msa_prof_begin(self.kid, self.max)
        if st != MSA_OK:
            raise MsaError(st, "msa_prof_begin")
        return self

    def __exit__(self, *exc):
        n = len(KERNELS)
        ms = (ctypes.c_float * n)()
        cnt = (ctypes.c_int * n)()
        st = lib().msa_prof_end(ms, cnt)
        if st != MSA_OK:
            raise MsaError(st, "msa_prof_end")
        self.per_kernel = {KERNELS[x]: (ms[x], cnt[x]) for x in range(n) if cnt[x] > 0}
        self.total_ms = sum(v[0] for v in self.per_kernel.values())
        self.launches = sum(v[1] for v in self.per_kernel.values())
        return False

    @property
    def avg_ms(self) -> float:
        return self.total_ms / max(1, self.launches)
