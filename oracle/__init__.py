"""fp64 CPU oracle of the MSA layer hot path — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (``learned_kv_block_amd``)
never imports it, and the oracle shares no code with the HIP kernels.

The arithmetic lives in ``msa_oracle.c`` (plain double-precision loops, one
query row at a time); this module only builds it with gcc and marshals numpy
arrays through ctypes. ``diagnostics.py`` holds the selector metrics (set
recall, teacher-mass coverage, relative output error).

Every oracle function here is pinned by CPU tests against values fixed by the
pages or by mathematics (worked examples, closed forms, library special
cases, brute force, finite differences); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmsa_ref.so")


class RefShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seqlen_kv", "seqlen_q", "q_start", "num_q_heads", "num_kv_heads",
        "head_dim", "idx_dim", "block_size", "topk", "dtype")]


def build(force: bool = False) -> None:
    """Compile the oracle with gcc (-O2, OpenMP over query rows)."""
    if force or not os.path.exists(_SO):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", _SO + ".tmp",
                               os.path.join(_HERE, "msa_oracle.c"), "-lm"])
        os.replace(_SO + ".tmp", _SO)


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        sp = ctypes.POINTER(RefShape)
        lib.msa_ref_topk_row.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
        lib.msa_ref_select.argtypes = [sp, P, P, P, I64, P, P, P, P, ctypes.c_int]
        lib.msa_ref_attn.argtypes = [sp, P, P, P, P, P, I64, P, P, ctypes.c_int]
        lib.msa_ref_kl_row.argtypes = [ctypes.c_int, I64, P, P, P, P, P, P, P]
        lib.msa_ref_kl.argtypes = [sp, P, P, P, P, P, P, I64, P, P, P, P, P, ctypes.c_int]
        lib.msa_ref_attn_bwd.argtypes = [sp, P, P, P, P, P, P, I64, P, P, P, ctypes.c_int]
        lib.msa_ref_idx_bwd.argtypes = [sp, P, P, P, P, ctypes.c_double, P, I64, P, P]
        lib.msa_ref_e4m3_encode.argtypes = [ctypes.c_double]
        lib.msa_ref_e4m3_encode.restype = ctypes.c_uint8
        lib.msa_ref_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.msa_ref_e4m3_decode.restype = ctypes.c_double
        lib.msa_ref_fp8_scale_exp.argtypes = [ctypes.c_double]
        lib.msa_ref_quantize_fp8.argtypes = [sp, P, P, I64, P, P, P, P, ctypes.c_int]
        lib.msa_ref_select_fp8.argtypes = [sp, P, P, P, P, P, I64, P, P, P, ctypes.c_int]
        for f in ("msa_ref_topk_row", "msa_ref_select", "msa_ref_attn", "msa_ref_kl_row",
                  "msa_ref_kl", "msa_ref_attn_bwd", "msa_ref_idx_bwd", "msa_ref_fp8_scale_exp",
                  "msa_ref_quantize_fp8", "msa_ref_select_fp8"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads of the oracle: every CPU this process may run on, at most 16 (the host
    share of one GPU on the measurement machines)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def shape_of(cfg) -> RefShape:
    """RefShape from any object with the MSA shape attributes (e.g. seeded_inputs.MsaConfig)."""
    return RefShape(cfg.batch, cfg.seqlen_kv, cfg.seqlen_q, cfg.q_start, cfg.num_q_heads,
                    cfg.num_kv_heads, cfg.head_dim, cfg.idx_dim, cfg.block_size, cfg.topk,
                    cfg.dtype)


def _raw(a: np.ndarray, dtype: int) -> np.ndarray:
    """Inputs are fp32 arrays (dtype 0) or uint16 bf16 bit patterns (dtype 1)."""
    want = np.float32 if dtype == 0 else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"oracle input must be {want.__name__} for dtype {dtype}, got {a.dtype}")
    return a


def _rows(shape: RefShape, rows):
    if rows is None:
        n = shape.batch * shape.seqlen_q
        return None, n
    r = _c(rows, np.int64)
    return r, r.shape[0]


def topk_row(M: Sequence[float], L: int, k: int):
    """Selection of one row of block scores M[0..L] (L = local block). Returns (ids, margin)."""
    M = _c(M, np.float64)
    ids = np.empty(k, dtype=np.int32)
    mg = np.zeros(1, dtype=np.float64)
    rc = _L().msa_ref_topk_row(_p(M), int(L), int(k), _p(ids), _p(mg))
    assert rc == 0
    return ids, float(mg[0])


def select(shape: RefShape, q_idx, k_idx, rows=None, want_scores=False, want_lse=False,
           want_margin=False):
    """ids [n, Hkv, k] (+ optional block scores / block LSE [n, Hkv, nb], margin [n, Hkv])."""
    q_idx = _raw(q_idx, shape.dtype)
    k_idx = _raw(k_idx, shape.dtype)
    r, n = _rows(shape, rows)
    nb = (shape.seqlen_kv + shape.block_size - 1) // shape.block_size
    H = shape.num_kv_heads
    ids = np.empty((n, H, shape.topk), dtype=np.int32)
    sc = np.empty((n, H, nb), dtype=np.float64) if want_scores else None
    bl = np.empty((n, H, nb), dtype=np.float64) if want_lse else None
    mg = np.empty((n, H), dtype=np.float64) if want_margin else None
    rc = _L().msa_ref_select(ctypes.byref(shape), _p(q_idx), _p(k_idx), _p(r), n, _p(ids),
                             _p(sc), _p(bl), _p(mg), threads())
    assert rc == 0, rc
    out = {"ids": ids}
    if want_scores:
        out["block_scores"] = sc
    if want_lse:
        out["block_lse"] = bl
    if want_margin:
        out["margin"] = mg
    return out


def attn(shape: RefShape, q, k, v, ids, rows=None):
    """(O [n, Hq, d], LSE [n, Hq]) in float64 on the support given by ids [n, Hkv, k]."""
    q = _raw(q, shape.dtype)
    k = _raw(k, shape.dtype)
    v = _raw(v, shape.dtype)
    ids = _c(ids, np.int32)
    r, n = _rows(shape, rows)
    out = np.empty((n, shape.num_q_heads, shape.head_dim), dtype=np.float64)
    lse = np.empty((n, shape.num_q_heads), dtype=np.float64)
    rc = _L().msa_ref_attn(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(ids), _p(r), n, _p(out),
                           _p(lse), threads())
    assert rc == 0, rc
    return out, lse


def kl_row(s_main, s_idx):
    """KL alignment of one row from explicit logits: s_main [G, n], s_idx [n].

    Returns dict(kl, dS, P, P_idx, lse_idx)."""
    s_main = _c(s_main, np.float64)
    s_idx = _c(s_idx, np.float64)
    G, n = s_main.shape
    kl = np.zeros(1)
    dS = np.empty(n)
    P = np.empty(n)
    Pi = np.empty(n)
    li = np.zeros(1)
    rc = _L().msa_ref_kl_row(G, n, _p(s_main), _p(s_idx), _p(kl), _p(dS), _p(P), _p(Pi), _p(li))
    assert rc == 0
    return {"kl": float(kl[0]), "dS": dS, "P": P, "P_idx": Pi, "lse_idx": float(li[0])}


def kl(shape: RefShape, q, k, q_idx, k_idx, ids, rows=None, want_dlogits=True, want_mass=False):
    """KL alignment: dict(kl_rows [n, Hkv], kl_mean, lse_idx [n, Hkv], dlogits [n, Hkv, k, Bk],
    block_mass [n, Hkv, k] when want_mass: teacher probability per slot's block)."""
    q = _raw(q, shape.dtype)
    k = _raw(k, shape.dtype)
    q_idx = _raw(q_idx, shape.dtype)
    k_idx = _raw(k_idx, shape.dtype)
    ids = _c(ids, np.int32)
    r, n = _rows(shape, rows)
    H = shape.num_kv_heads
    klr = np.empty((n, H), dtype=np.float64)
    li = np.empty((n, H), dtype=np.float64)
    dl = np.empty((n, H, shape.topk, shape.block_size), dtype=np.float64) if want_dlogits else None
    bm = np.empty((n, H, shape.topk), dtype=np.float64) if want_mass else None
    mean = np.zeros(1)
    rc = _L().msa_ref_kl(ctypes.byref(shape), _p(q), _p(k), _p(q_idx), _p(k_idx), _p(ids), _p(r),
                         n, _p(klr), _p(dl), _p(li), _p(mean), _p(bm), threads())
    assert rc == 0, rc
    out = {"kl_rows": klr, "kl_mean": float(mean[0]), "lse_idx": li}
    if want_dlogits:
        out["dlogits"] = dl
    if want_mass:
        out["block_mass"] = bm
    return out


def dense_shape(shape: RefShape) -> RefShape:
    """The same shape with k = every block: the warm-up stage's full causal context."""
    nb = (shape.seqlen_kv + shape.block_size - 1) // shape.block_size
    return RefShape(shape.batch, shape.seqlen_kv, shape.seqlen_q, shape.q_start,
                    shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.idx_dim,
                    shape.block_size, nb, shape.dtype)


def dense_ids(shape: RefShape, rows=None) -> np.ndarray:
    """[n, Hkv, nb] block lists 0..floor(i/Bk) (then -1) of the listed rows: with
    dense_shape(shape) the support of every row is its full causal context."""
    nb = (shape.seqlen_kv + shape.block_size - 1) // shape.block_size
    r = np.arange(shape.batch * shape.seqlen_q) if rows is None else np.asarray(rows, np.int64)
    i = shape.q_start + r % max(shape.seqlen_q, 1)
    blk = np.arange(nb)[None, :]
    ids = np.where(blk <= (i // shape.block_size)[:, None], blk, -1).astype(np.int32)
    return np.ascontiguousarray(np.repeat(ids[:, None, :], shape.num_kv_heads, axis=1))


def attn_bwd(shape: RefShape, q, k, v, ids, dout, rows=None, want_kv=True):
    """Gradients with the selection fixed: (dq [n, Hq, d], dk, dv [B, N, Hkv, d]) in float64.

    q and dout are compact [n, Hq, d] in the input dtype; dk/dv sum over the listed rows
    (None when want_kv is False)."""
    q = _raw(q, shape.dtype)
    k = _raw(k, shape.dtype)
    v = _raw(v, shape.dtype)
    dout = _raw(dout, shape.dtype)
    ids = _c(ids, np.int32)
    r, n = _rows(shape, rows)
    d = shape.head_dim
    dq = np.empty((n, shape.num_q_heads, d), dtype=np.float64)
    kv_shape = (shape.batch, shape.seqlen_kv, shape.num_kv_heads, d)
    dk = np.empty(kv_shape, dtype=np.float64) if want_kv else None
    dv = np.empty(kv_shape, dtype=np.float64) if want_kv else None
    rc = _L().msa_ref_attn_bwd(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(ids), _p(dout), _p(r),
                               n, _p(dq), _p(dk), _p(dv), threads())
    assert rc == 0, rc
    return dq, dk, dv


def idx_bwd(shape: RefShape, q_idx, k_idx, ids, dlogits, coef=1.0, rows=None):
    """(dq_idx [n, Hkv, d_idx], dk_idx [B, N, d_idx]) in float64 from dlogits [n, Hkv, k, Bk]."""
    q_idx = _raw(q_idx, shape.dtype)
    k_idx = _raw(k_idx, shape.dtype)
    ids = _c(ids, np.int32)
    dl = _c(dlogits, np.float64)
    r, n = _rows(shape, rows)
    dq = np.empty((n, shape.num_kv_heads, shape.idx_dim), dtype=np.float64)
    dk = np.empty((shape.batch, shape.seqlen_kv, shape.idx_dim), dtype=np.float64)
    rc = _L().msa_ref_idx_bwd(ctypes.byref(shape), _p(q_idx), _p(k_idx), _p(ids), _p(dl),
                              float(coef), _p(r), n, _p(dq), _p(dk))
    assert rc == 0, rc
    return dq, dk


# ----------------------------------------------------------------------- FP8 index scoring


def e4m3_encode(values) -> np.ndarray:
    """OCP E4M3 codes (uint8) of values with |v| <= 448: nearest value, ties to the even code."""
    v = np.asarray(values, dtype=np.float64).ravel()
    f = _L().msa_ref_e4m3_encode
    return np.array([f(float(x)) for x in v], dtype=np.uint8).reshape(np.shape(values))


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).ravel()
    f = _L().msa_ref_e4m3_decode
    return np.array([f(int(x)) for x in c], dtype=np.float64).reshape(np.shape(codes))


def fp8_scale_exp(amax: float) -> int:
    """Smallest e with amax <= 448 * 2^e (0 for amax = 0)."""
    return int(_L().msa_ref_fp8_scale_exp(float(amax)))


def quantize_fp8(shape: RefShape, q_idx, k_idx=None):
    """dict(q8 [n, Hkv, d_idx] uint8, q_exp [n, Hkv] int32, and with k_idx: k8 [B, N, d_idx],
    k_exp [B, nb]) for compact q_idx rows [n, Hkv, d_idx]."""
    q_idx = _raw(q_idx, shape.dtype)
    n = q_idx.shape[0]
    H, di = shape.num_kv_heads, shape.idx_dim
    nb = (shape.seqlen_kv + shape.block_size - 1) // shape.block_size
    q8 = np.empty((n, H, di), dtype=np.uint8)
    qe = np.empty((n, H), dtype=np.int32)
    k8 = ke = None
    if k_idx is not None:
        k_idx = _raw(k_idx, shape.dtype)
        k8 = np.zeros((shape.batch, shape.seqlen_kv, di), dtype=np.uint8)
        ke = np.empty((shape.batch, nb), dtype=np.int32)
    rc = _L().msa_ref_quantize_fp8(ctypes.byref(shape), _p(q_idx), _p(k_idx), n, _p(q8), _p(qe),
                                   _p(k8), _p(ke), threads())
    assert rc == 0, rc
    out = {"q8": q8, "q_exp": qe}
    if k_idx is not None:
        out.update(k8=k8, k_exp=ke)
    return out


def select_fp8(shape: RefShape, q8, q_exp, k8, k_exp, rows=None, want_scores=False,
               want_margin=False):
    """Selection on the FP8 index logits: ids [n, Hkv, k] (+ block scores, margin)."""
    q8, qe = _c(q8, np.uint8), _c(q_exp, np.int32)
    k8, ke = _c(k8, np.uint8), _c(k_exp, np.int32)
    r, n = _rows(shape, rows)
    nb = (shape.seqlen_kv + shape.block_size - 1) // shape.block_size
    H = shape.num_kv_heads
    ids = np.empty((n, H, shape.topk), dtype=np.int32)
    sc = np.empty((n, H, nb), dtype=np.float64) if want_scores else None
    mg = np.empty((n, H), dtype=np.float64) if want_margin else None
    rc = _L().msa_ref_select_fp8(ctypes.byref(shape), _p(q8), _p(qe), _p(k8), _p(ke), _p(r), n,
                                 _p(ids), _p(sc), _p(mg), threads())
    assert rc == 0, rc
    out = {"ids": ids}
    if want_scores:
        out["block_scores"] = sc
    if want_margin:
        out["margin"] = mg
    return out
