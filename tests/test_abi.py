"""C ABI: the library loads, exports every entry point declared in include/msa.h,
and rejects bad arguments on the host before touching the device (CPU only)."""
import ctypes
import os
import re

import pytest

import learned_kv_block_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails before any launch


def declared_functions():
    src = open(os.path.join(ROOT, "include", "msa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = msa.lib()
    names = declared_functions()
    assert set(names) == set(msa.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def shape(**kw):
    base = dict(batch=1, seqlen_kv=1024, seqlen_q=1024, q_start=0, num_q_heads=64,
                num_kv_heads=4, head_dim=128, idx_dim=64, topk=16, dtype=msa.MSA_BF16)
    base.update(kw)
    return msa.make_shape(**base)


def select(sh, ws=None, nws=0, ids=FAKE, qi=FAKE, ki=FAKE):
    return msa.lib().msa_select(ctypes.byref(sh), qi, ki, ids, None, None, ws, nws, None)


def test_status_strings():
    for s in range(6):
        assert msa.status_string(s)


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
    # partial outputs: slots * G * d * 2 bytes (bf16) dominate the attention workspace
    assert msa.workspace_size(big, msa.MSA_OP_ATTN) >= 131072 * 4 * 16 * 16 * 128 * 2
    assert msa.workspace_size(small, msa.MSA_OP_ATTN) < msa.workspace_size(big, msa.MSA_OP_ATTN)
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
