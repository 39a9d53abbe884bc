"""C ABI: the library loads, exports every entry point declared in include/msa.h,
and rejects bad arguments on the host before touching the device (CPU only)."""
import ctypes
import os
import re

import pytest

import learned_kv_block_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails before any launch


def declared_functions(header="msa.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    """libmsa.so exports what msa.h declares and holds no timing hook; libmsa_timed.so (the
    measurement build) exports that plus what msa_timing.h declares."""
    L = msa.lib()
    names = declared_functions()
    assert set(names) == set(msa.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    timing = declared_functions("msa_timing.h")
    assert set(timing) == set(msa.TIMING_EXPORTS)
    for n in timing:
        assert not hasattr(L, n), f"the product library must not export {n}"
    T = ctypes.CDLL(msa.TIMED_LIB_PATH)
    for n in names + timing:
        assert hasattr(T, n), n


def shape(**kw):
    base = dict(batch=1, seqlen_kv=1024, seqlen_q=1024, q_start=0, num_q_heads=64,
                num_kv_heads=4, head_dim=128, idx_dim=64, topk=16, dtype=msa.MSA_BF16)
    base.update(kw)
    return msa.make_shape(**base)


def select(sh, ws=None, nws=0, ids=FAKE, qi=FAKE, ki=FAKE):
    return msa.lib().msa_select(ctypes.byref(sh), qi, ki, ids, None, None, ws, nws, None)


def test_status_strings():
    for s in range(7):
        assert msa.status_string(s)


def test_noalloc_rejects_on_host():
    """msa_attn_fwd_noalloc: NULL pointers, and workloads whose workspace exceeds the fixed
    64 MiB scratch, are rejected before anything is launched."""
    L = msa.lib()
    small = shape(batch=16, seqlen_kv=8192, seqlen_q=1, q_start=8191)
    assert msa.workspace_size(small, msa.MSA_OP_ATTN) <= msa.NOALLOC_SCRATCH_BYTES
    assert L.msa_attn_fwd_noalloc(ctypes.byref(small), FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                  None) == msa.MSA_ERR_NULL
    big = shape(seqlen_kv=8192, seqlen_q=8192)
    assert msa.workspace_size(big, msa.MSA_OP_ATTN) > msa.NOALLOC_SCRATCH_BYTES
    assert L.msa_attn_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  None) == msa.MSA_ERR_SCRATCH
    assert "scratch" in msa.status_string(msa.MSA_ERR_SCRATCH)


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=63), msa.MSA_ERR_SHAPE),
    (dict(q_start=1, seqlen_q=1024), msa.MSA_ERR_SHAPE),
    (dict(topk=0), msa.MSA_ERR_SHAPE),
    (dict(batch=-1), msa.MSA_ERR_SHAPE),
    (dict(dtype=7), msa.MSA_ERR_SHAPE),
    (dict(head_dim=96), msa.MSA_ERR_UNSUPPORTED),
    (dict(idx_dim=128), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_q_heads=128, num_kv_heads=4), msa.MSA_ERR_UNSUPPORTED),  # G = 32
    (dict(topk=33), msa.MSA_ERR_UNSUPPORTED),
    (dict(seqlen_kv=300000, seqlen_q=1), msa.MSA_ERR_UNSUPPORTED),
    (dict(num_q_heads=48, num_kv_heads=3), msa.MSA_ERR_UNSUPPORTED),
])
def test_shape_validation(kw, status):
    sh = shape(**kw)
    assert select(sh) == status
    assert msa.workspace_size(sh, msa.MSA_OP_ATTN) == 0


def test_null_and_workspace_errors():
    L = msa.lib()
    sh = shape()
    assert L.msa_select(None, FAKE, FAKE, FAKE, None, None, None, 0, None) == msa.MSA_ERR_NULL
    assert select(sh, ids=None) == msa.MSA_ERR_NULL
    assert select(sh, qi=None) == msa.MSA_ERR_NULL
    need = msa.workspace_size(sh, msa.MSA_OP_SELECT)
    assert need == 1024 * 4 * 8 * 4
    assert select(sh) == msa.MSA_ERR_WORKSPACE
    assert select(sh, ws=FAKE, nws=need - 1) == msa.MSA_ERR_WORKSPACE
    assert select(sh, ws=ctypes.c_void_p(0x100010), nws=need) == msa.MSA_ERR_WORKSPACE  # alignment
    # attention / KL: NULL outputs and small workspaces
    assert L.msa_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40,
                          None) == msa.MSA_ERR_NULL
    na = msa.workspace_size(sh, msa.MSA_OP_ATTN)
    assert na > 0
    assert L.msa_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, na - 1,
                          None) == msa.MSA_ERR_WORKSPACE
    nk = msa.workspace_size(sh, msa.MSA_OP_KL)
    assert L.msa_kl_align(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                          None, FAKE, nk, None) == msa.MSA_ERR_NULL
    assert L.msa_kl_align(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          None, FAKE, nk - 1, None) == msa.MSA_ERR_WORKSPACE
    # misaligned tensor pointers
    assert select(sh, qi=ctypes.c_void_p(0x100004), ws=FAKE, nws=need) == msa.MSA_ERR_SHAPE


def test_empty_workloads_are_noops():
    sh = shape(seqlen_q=0)
    assert select(sh, ids=None, qi=None, ki=None) == msa.MSA_OK
    sh = shape(batch=0)
    assert msa.lib().msa_attn_fwd(ctypes.byref(sh), None, None, None, None, None, None, None, 0,
                                  None) == msa.MSA_OK


def test_workspace_sizes_scale_with_the_workload():
    small = shape(seqlen_kv=8192, seqlen_q=8192)
    big = shape(seqlen_kv=131072, seqlen_q=131072)
    # partial outputs: slots * G * d * 2 bytes (bf16) dominate the attention workspace;
    # a sequence of more than 32768 queries runs the attention in 32768-query windows
    # that share one window's workspace, the same as a 32768-query call's
    window = shape(seqlen_kv=131072, seqlen_q=32768)
    assert msa.workspace_size(big, msa.MSA_OP_ATTN) >= 32768 * 4 * 16 * 16 * 128 * 2
    assert msa.workspace_size(big, msa.MSA_OP_ATTN) == msa.workspace_size(window, msa.MSA_OP_ATTN)
    assert msa.workspace_size(small, msa.MSA_OP_ATTN) < msa.workspace_size(big, msa.MSA_OP_ATTN)
    # the other calls still scale with the whole workload
    assert msa.workspace_size(big, msa.MSA_OP_SELECT) == 131072 * 4 * 1024 * 4
    assert msa.workspace_size(big, 7) == 0


def test_dense_calls_validate_on_host():
    """msa_dense_lse / msa_kl_dense / msa_block_recall reject NULL outputs, misaligned inputs
    and fp32 with head_dim 128 before any launch."""
    L = msa.lib()
    sh = shape()
    assert L.msa_dense_lse(ctypes.byref(sh), FAKE, FAKE, None, None) == msa.MSA_ERR_NULL
    assert L.msa_dense_lse(ctypes.byref(sh), ctypes.c_void_p(0x100002), FAKE, FAKE,
                           None) == msa.MSA_ERR_SHAPE
    f32 = shape(dtype=msa.MSA_F32)
    assert L.msa_dense_lse(ctypes.byref(f32), FAKE, FAKE, FAKE, None) == msa.MSA_ERR_UNSUPPORTED
    assert L.msa_kl_dense(ctypes.byref(f32), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          None, None) == msa.MSA_ERR_UNSUPPORTED
    assert L.msa_kl_dense(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                          None, None) == msa.MSA_ERR_NULL
    assert L.msa_kl_dense(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                          None, None) == msa.MSA_ERR_NULL
    assert L.msa_block_recall(ctypes.byref(sh), FAKE, None, FAKE, FAKE, None,
                              None) == msa.MSA_ERR_NULL
    assert L.msa_block_recall(ctypes.byref(shape(topk=40)), FAKE, FAKE, FAKE, FAKE, None,
                              None) == msa.MSA_ERR_UNSUPPORTED


def test_fp8_calls_validate_on_host():
    L = msa.lib()
    sh = shape()
    assert L.msa_index_quantize_fp8(ctypes.byref(sh), FAKE, FAKE, None, None, None, None,
                                    None) == msa.MSA_ERR_NULL
    assert L.msa_index_quantize_fp8(ctypes.byref(sh), None, FAKE, FAKE, FAKE, None, None,
                                    None) == msa.MSA_ERR_NULL
    assert L.msa_index_quantize_fp8(ctypes.byref(sh), FAKE, FAKE, ctypes.c_void_p(0x100004),
                                    FAKE, None, None, None) == msa.MSA_ERR_SHAPE
    assert L.msa_select_fp8(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, None, None, None, None, 0,
                            None) == msa.MSA_ERR_NULL
    assert L.msa_select_fp8(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0,
                            None) == msa.MSA_ERR_WORKSPACE
    assert L.msa_select_fp8(ctypes.byref(shape(topk=33)), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                            None, None, 0, None) == msa.MSA_ERR_UNSUPPORTED


def test_dense_bwd_validates_on_host():
    L = msa.lib()
    sh = shape()
    need = msa.workspace_size(sh, msa.MSA_OP_KL_DENSE_BWD)
    assert need >= 1024 * 4 * 1024 * 2  # one chunk of bf16 dS rows
    args = [ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE, FAKE, FAKE,
            None, FAKE, FAKE]
    assert L.msa_kl_dense_bwd(*args, None, 0, None) == msa.MSA_ERR_WORKSPACE
    bad = list(args)
    bad[11] = None  # dq_idx
    assert L.msa_kl_dense_bwd(*bad, FAKE, need, None) == msa.MSA_ERR_NULL
    bad = list(args)
    bad[8] = None  # kl_rows NULL with kl_mean given
    assert L.msa_kl_dense_bwd(*bad, FAKE, need, None) == msa.MSA_ERR_NULL


# ------------------------------------------------------------- binding: argument checks
# The library sees raw pointers, so the binding must reject every shape, dtype or size
# mismatch before a call: a wrong size would make the kernels read or write out of bounds.
# These run on CPU tensors; the device check comes last, so a well-formed argument list
# reaches it and fails with "device tensor" instead.

import torch  # noqa: E402

BF = torch.bfloat16


def _attn_args(B=1, Nq=256, N=256, Hq=8, Hkv=2, D=64, K=4, dt=BF):
    return dict(q=torch.zeros(B, Nq, Hq, D, dtype=dt), k=torch.zeros(B, N, Hkv, D, dtype=dt),
                v=torch.zeros(B, N, Hkv, D, dtype=dt),
                block_ids=torch.zeros(B, Nq, Hkv, K, dtype=torch.int32))


@pytest.mark.parametrize("change,match", [
    (dict(block_ids=torch.zeros(1, 256, 2, 4, dtype=torch.int64)), "int32"),
    (dict(k=torch.zeros(1, 256, 2, 64, dtype=torch.float32)), "bfloat16"),
    (dict(v=torch.zeros(1, 128, 2, 64, dtype=BF)), "dimension 1"),
    (dict(k=torch.zeros(1, 256, 2, 128, dtype=BF)), "dimension 3"),
    (dict(block_ids=torch.zeros(1, 256, 4, 4, dtype=torch.int32)), "dimension 2"),
    (dict(block_ids=torch.zeros(2, 256, 2, 4, dtype=torch.int32)), "dimension 0"),
    (dict(q=torch.zeros(1, 256, 8, 64, dtype=BF).transpose(1, 2).contiguous().transpose(1, 2)),
     "contiguous"),
])
def test_attn_fwd_rejects_mismatched_arguments(change, match):
    a = _attn_args()
    a.update(change)
    with pytest.raises(ValueError, match=match):
        msa.msa_attn_fwd(**a)


def test_attn_fwd_rejects_bad_outputs_and_cpu_tensors():
    a = _attn_args()
    with pytest.raises(ValueError, match="float32"):
        msa.msa_attn_fwd(**a, lse=torch.zeros(1, 256, 8, dtype=BF))
    with pytest.raises(ValueError, match="dimension 2"):
        msa.msa_attn_fwd(**a, out=torch.zeros(1, 256, 4, 64, dtype=BF))
    with pytest.raises(ValueError, match="device tensor"):
        msa.msa_attn_fwd(**a)


def test_select_kl_bwd_recall_fp8_reject_mismatches():
    qi = torch.zeros(1, 256, 2, 32, dtype=BF)
    with pytest.raises(ValueError, match="dimension 2"):
        msa.msa_select(qi, torch.zeros(1, 256, 64, dtype=BF), 4)
    with pytest.raises(ValueError, match="bfloat16"):
        msa.msa_select(qi, torch.zeros(1, 256, 32, dtype=torch.float32), 4)
    a = _attn_args()
    ki = torch.zeros(1, 256, 32, dtype=BF)
    lse = torch.zeros(1, 256, 8, dtype=torch.float32)
    with pytest.raises(ValueError, match="dimension 1"):  # k_idx shorter than k
        msa.msa_kl_align(a["q"], a["k"], qi, torch.zeros(1, 128, 32, dtype=BF), a["block_ids"],
                         lse)
    with pytest.raises(ValueError, match="dimension 2"):  # lse per group instead of per head
        msa.msa_kl_align(a["q"], a["k"], qi, ki, a["block_ids"],
                         torch.zeros(1, 256, 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="q_idx.*dimension 2"):  # q_idx per head, not per group
        msa.msa_kl_align(a["q"], a["k"], torch.zeros(1, 256, 8, 32, dtype=BF), ki,
                         a["block_ids"], lse)
    with pytest.raises(ValueError, match="dout"):
        msa.msa_attn_bwd(a["q"], a["k"], a["v"], a["block_ids"], a["q"], lse,
                         torch.zeros(1, 256, 8, 32, dtype=BF))
    with pytest.raises(ValueError, match="dimension 4"):
        msa.msa_idx_bwd(qi, ki, a["block_ids"], torch.zeros(1, 256, 2, 4, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="float32"):
        msa.msa_block_recall(torch.zeros(1, 256, 2, 2, dtype=BF), a["block_ids"])
    with pytest.raises(ValueError, match="int32"):
        msa.msa_select_fp8(torch.zeros(1, 256, 2, 32, dtype=torch.uint8),
                           torch.zeros(1, 256, 2, dtype=torch.int64),
                           torch.zeros(1, 256, 32, dtype=torch.uint8),
                           torch.zeros(1, 2, dtype=torch.int32), 4)
    with pytest.raises(ValueError, match="dimension 1"):  # one exponent per 128-token block
        msa.msa_select_fp8(torch.zeros(1, 256, 2, 32, dtype=torch.uint8),
                           torch.zeros(1, 256, 2, dtype=torch.int32),
                           torch.zeros(1, 256, 32, dtype=torch.uint8),
                           torch.zeros(1, 3, dtype=torch.int32), 4)
