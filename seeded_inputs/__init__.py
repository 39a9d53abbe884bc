"""Seeded synthetic inputs for the MSA layer workloads.

Test and benchmark infrastructure shared by the oracle side and the GPU side;
it holds none of the method's arithmetic. Every value comes from the
counter-based generator of ``msa_gen.h`` (SplitMix64 hashing, Irwin-Hall(12)
approximation of N(0,1), an affine scale/shift in double, IEEE rounding to the
storage type), so any row can be rebuilt on its own and the host and device
builds give identical bits.

Workloads (shapes of the MSA main recipe: Hq=64, Hkv=4, Bk=128, k=16):

===================  ==========================================================
name                 what
===================  ==========================================================
tiny_f32_n1024       batch 1, N=1024, Hq=4, Hkv=2, d=64, d_idx=32, k=4, fp32,
                     unscaled N(0,1)
main_n8192           batch 1, N=8192, Hq=64, Hkv=4, d=128, d_idx=64, k=16, bf16,
                     N(0,1)/sqrt(2)
train_b2_n32768      as main at batch 2, N=32768 (+ KL alignment pass)
skewed_n131072       as main at N=131072, skewed routing: K_idx rows of block 0
                     and of 64 seeded hot blocks, and a seeded half of the
                     Q_idx rows, get +3 sigma along one shared unit direction
decode_b64_n131072   64 sequences with 131072-token caches, one query each at
                     position N-1
===================  ==========================================================
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SO = os.path.join(_HERE, "libmsa_gen.so")
_DEV_SO = os.path.join(_HERE, "libmsa_gen_hip.so")

F32, BF16 = 0, 1

# Tensor ids of the generator streams.
TID = {"q": 1, "k": 2, "v": 3, "q_idx": 4, "k_idx": 5, "hot": 6, "dir": 7, "boost": 8,
       "dout": 9}


@dataclasses.dataclass(frozen=True)
class MsaConfig:
    name: str
    batch: int
    seqlen_kv: int
    seqlen_q: int
    q_start: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    idx_dim: int
    block_size: int
    topk: int
    dtype: int  # F32 or BF16
    scale: float  # multiplies the N(0,1) draw
    seed: int
    skew: bool = False
    hot_blocks: int = 64
    boost_sigmas: float = 3.0
    with_kl: bool = False

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_blocks(self) -> int:
        return (self.seqlen_kv + self.block_size - 1) // self.block_size

    def replace(self, **kw) -> "MsaConfig":
        return dataclasses.replace(self, **kw)

    # [rows, cols] views of every tensor
    def view(self, name: str):
        B, N, Nq = self.batch, self.seqlen_kv, self.seqlen_q
        if name in ("q", "dout"):
            return B * Nq, self.num_q_heads * self.head_dim
        if name in ("k", "v"):
            return B * N, self.num_kv_heads * self.head_dim
        if name == "q_idx":
            return B * Nq * self.num_kv_heads, self.idx_dim
        if name == "k_idx":
            return B * N, self.idx_dim
        raise KeyError(name)

    def shape(self, name: str):
        B, N, Nq = self.batch, self.seqlen_kv, self.seqlen_q
        if name in ("q", "dout"):
            return (B, Nq, self.num_q_heads, self.head_dim)
        if name in ("k", "v"):
            return (B, N, self.num_kv_heads, self.head_dim)
        if name == "q_idx":
            return (B, Nq, self.num_kv_heads, self.idx_dim)
        if name == "k_idx":
            return (B, N, self.idx_dim)
        raise KeyError(name)


_INV_SQRT2 = 0.70710678118654752440

CONFIGS: Dict[str, MsaConfig] = {
    "tiny_f32_n1024": MsaConfig("tiny_f32_n1024", 1, 1024, 1024, 0, 4, 2, 64, 32, 128, 4,
                                F32, 1.0, 1, with_kl=True),
    "main_n8192": MsaConfig("main_n8192", 1, 8192, 8192, 0, 64, 4, 128, 64, 128, 16,
                            BF16, _INV_SQRT2, 2),
    "train_b2_n32768": MsaConfig("train_b2_n32768", 2, 32768, 32768, 0, 64, 4, 128, 64, 128,
                                 16, BF16, _INV_SQRT2, 3, with_kl=True),
    "skewed_n131072": MsaConfig("skewed_n131072", 1, 131072, 131072, 0, 64, 4, 128, 64, 128,
                                16, BF16, _INV_SQRT2, 4, skew=True),
    "decode_b64_n131072": MsaConfig("decode_b64_n131072", 64, 131072, 1, 131071, 64, 4, 128,
                                    64, 128, 16, BF16, _INV_SQRT2, 5),
}


# --------------------------------------------------------------------------- build / load

def build(force: bool = False) -> None:
    """Compile the host (gcc) and device (hipcc, gfx950) generator libraries in-tree."""
    hdr = os.path.join(_HERE, "msa_gen.h")
    host_src = os.path.join(_HERE, "gen_host.c")
    dev_src = os.path.join(_HERE, "gen_device.hip")
    if force or not os.path.exists(_HOST_SO):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared",
                               "-fPIC", "-o", _HOST_SO + ".tmp", host_src, "-I", _HERE])
        os.replace(_HOST_SO + ".tmp", _HOST_SO)
    if force or not os.path.exists(_DEV_SO):
        hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
        subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O3", "-ffp-contract=off",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-shared", "-fPIC", "-o", _DEV_SO + ".tmp", dev_src, "-I", _HERE],
                              stderr=subprocess.DEVNULL)
        os.replace(_DEV_SO + ".tmp", _DEV_SO)
    del hdr


_host_lib = None
_dev_lib = None


def _host():
    global _host_lib
    if _host_lib is None:
        if not os.path.exists(_HOST_SO):
            build()
        lib = ctypes.CDLL(_HOST_SO)
        lib.msa_gen_fill_host.restype = ctypes.c_int
        lib.msa_gen_fill_host.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.msa_gen_bits_host.restype = ctypes.c_int
        lib.msa_gen_bits_host.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                          ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
        lib.msa_gen_normals_host.restype = ctypes.c_int
        lib.msa_gen_normals_host.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                                             ctypes.c_int64, ctypes.c_void_p]
        _host_lib = lib
    return _host_lib


def _dev():
    global _dev_lib
    if _dev_lib is None:
        if not os.path.exists(_DEV_SO):
            build()
        lib = ctypes.CDLL(_DEV_SO)
        lib.msa_gen_fill_device.restype = ctypes.c_int
        lib.msa_gen_fill_device.argtypes = [
            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        _dev_lib = lib
    return _dev_lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data if a is not None else None


def host_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


# --------------------------------------------------------------------------- seeded draws

def bits(seed: int, tid: int, e0: int, n: int, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Raw 64-bit hashes of elements e0..e0+n-1 (or of the listed element indices)."""
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.shape[0]
    out = np.empty(n, dtype=np.uint64)
    if n:
        rc = _host().msa_gen_bits_host(seed, tid, _ptr(rows), e0, n, _ptr(out))
        assert rc == 0
    return out


def normals_f64(seed: int, tid: int, e0: int, n: int) -> np.ndarray:
    """The generator's unscaled, unrounded N(0,1) draws e0..e0+n-1 in double."""
    out = np.empty(n, dtype=np.float64)
    if n:
        rc = _host().msa_gen_normals_host(seed, tid, e0, n, _ptr(out))
        assert rc == 0
    return out


def hot_block_list(cfg: MsaConfig) -> np.ndarray:
    """Block 0 plus `hot_blocks` distinct blocks drawn uniformly from 1..nb-1."""
    nb = cfg.num_blocks
    want = min(cfg.hot_blocks, nb - 1)
    chosen = []
    e = 0
    while len(chosen) < want:
        draws = bits(cfg.seed, TID["hot"], e, 256)
        e += 256
        for d in draws:
            b = 1 + int(d % np.uint64(nb - 1))
            if b not in chosen:
                chosen.append(b)
                if len(chosen) == want:
                    break
    return np.array([0] + sorted(chosen), dtype=np.int64)


def skew_shift(cfg: MsaConfig) -> np.ndarray:
    """boost_sigmas * sigma * u, with u a seeded unit vector in R^{d_idx} and sigma = cfg.scale."""
    g = normals_f64(cfg.seed, TID["dir"], 0, cfg.idx_dim)
    u = g / math.sqrt(float(np.dot(g, g)))
    return (cfg.boost_sigmas * cfg.scale) * u


def q_idx_boost_flags(cfg: MsaConfig, rows: np.ndarray) -> np.ndarray:
    """Seeded boost bit (probability 1/2) of Q_idx view rows (flat (b, t, r) indices)."""
    return (bits(cfg.seed, TID["boost"], 0, 0, rows=rows) & np.uint64(1)).astype(np.uint8)


def k_idx_boost_flags(cfg: MsaConfig, rows: np.ndarray) -> np.ndarray:
    """1 for K_idx view rows (flat (b, j) indices) whose token lies in a hot block."""
    hot = np.zeros(cfg.num_blocks, dtype=np.uint8)
    hot[hot_block_list(cfg)] = 1
    tok = np.asarray(rows, dtype=np.int64) % cfg.seqlen_kv
    return hot[tok // cfg.block_size]


def _flags_for(cfg: MsaConfig, name: str, rows: np.ndarray) -> Optional[np.ndarray]:
    if not cfg.skew:
        return None
    if name == "k_idx":
        return np.ascontiguousarray(k_idx_boost_flags(cfg, rows))
    if name == "q_idx":
        return np.ascontiguousarray(q_idx_boost_flags(cfg, rows))
    return None


# --------------------------------------------------------------------------- host tensors

def host_view_rows(cfg: MsaConfig, name: str, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Rows of the [rows, cols] view of tensor `name` as a numpy array.

    float32 for fp32 workloads, uint16 (bf16 bit patterns) for bf16 workloads.
    rows=None returns the whole tensor.
    """
    total, ncols = cfg.view(name)
    if rows is None:
        rows_a = np.arange(total, dtype=np.int64)
    else:
        rows_a = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows_a.shape[0]
    out = np.empty((n, ncols), dtype=np.float32 if cfg.dtype == F32 else np.uint16)
    flags = _flags_for(cfg, name, rows_a)
    shift = np.ascontiguousarray(skew_shift(cfg)) if flags is not None else None
    if n:
        rc = _host().msa_gen_fill_host(cfg.seed, TID[name], cfg.dtype, ncols,
                                       _ptr(rows_a), 0, n, cfg.scale, _ptr(shift), _ptr(flags),
                                       _ptr(out), host_threads())
        assert rc == 0, rc
    return out


def host_tensor(cfg: MsaConfig, name: str) -> np.ndarray:
    return host_view_rows(cfg, name).reshape(cfg.shape(name))


def host_query_rows(cfg: MsaConfig, name: str, qrows: Sequence[int]) -> np.ndarray:
    """q or q_idx for the listed query rows (flat b*Nq + t), compact [n, heads, dim]."""
    qrows = np.asarray(qrows, dtype=np.int64)
    if name in ("q", "dout"):
        return host_view_rows(cfg, name, qrows).reshape(qrows.shape[0], cfg.num_q_heads,
                                                          cfg.head_dim)
    if name == "q_idx":
        H = cfg.num_kv_heads
        vr = (qrows[:, None] * H + np.arange(H)[None, :]).reshape(-1)
        return host_view_rows(cfg, "q_idx", vr).reshape(qrows.shape[0], H, cfg.idx_dim)
    raise KeyError(name)


def host_batch_rows(cfg: MsaConfig, name: str, batches: Sequence[int]) -> np.ndarray:
    """k, v or k_idx for the listed batch entries only, [len(batches), N, ...]."""
    N = cfg.seqlen_kv
    rows = np.concatenate([np.arange(b * N, (b + 1) * N, dtype=np.int64) for b in batches])
    shp = cfg.shape(name)
    return host_view_rows(cfg, name, rows).reshape((len(batches),) + shp[1:])


# --------------------------------------------------------------------------- device tensors

def device_tensor(cfg: MsaConfig, name: str, device="cuda"):
    """The whole tensor generated on the GPU (torch, bf16 or fp32), bit-identical to the host."""
    import torch

    total, ncols = cfg.view(name)
    tdtype = torch.float32 if cfg.dtype == F32 else torch.bfloat16
    out = torch.empty(cfg.shape(name), dtype=tdtype, device=device)
    if total == 0:
        return out
    flags_t = shift_t = None
    if cfg.skew and name in ("q_idx", "k_idx"):
        flags = _flags_for(cfg, name, np.arange(total, dtype=np.int64))
        flags_t = torch.from_numpy(np.ascontiguousarray(flags)).to(device)
        shift_t = torch.from_numpy(np.ascontiguousarray(skew_shift(cfg))).to(device)
    stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = _dev().msa_gen_fill_device(cfg.seed, TID[name], cfg.dtype, ncols, 0, total, cfg.scale,
                                    shift_t.data_ptr() if shift_t is not None else None,
                                    flags_t.data_ptr() if flags_t is not None else None,
                                    out.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError(f"msa_gen_fill_device failed ({rc})")
    if flags_t is not None:
        # keep the small helper tensors alive until the fill has run
        torch.cuda.current_stream(out.device).synchronize()
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(cfg: MsaConfig, a: np.ndarray) -> np.ndarray:
    return a if cfg.dtype == F32 else bf16_bits_to_f32(a)
