"""Results must not depend on what the caller's workspace held before the call.

Each call runs once on a zeroed workspace and then twice on the same workspace with a float
region filled with 0xFF bytes (NaN in fp32 and bf16), and the outputs must be bit-identical
and free of NaN. Only regions that hold float data are filled (the selection's block-score
matrix, the backward kernels' fp32 dK/dV and dk_idx slabs, which are the last region of
their workspaces, and the whole workspace of the full-context KL backward), so an index or
count is never poisoned: a read of memory that the call did not write shows up as a NaN or a
changed bit, never as an access out of range.
The slab sizes follow the library's layout: one 128-key slab per (batch, group, block) bucket
plus two per persistent workgroup (at most 512 workgroups); the attention backward keeps two
32-row tiles of (dK, dV) per slab, the index backward one [128][d_idx] tile.
"""
import pytest
import torch

import seeded_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu


def _same(tag, ref, got):
    for i, (a, b) in enumerate(zip(ref, got)):
        assert not bool(torch.isnan(b.float()).any()), f"{tag}[{i}]: NaN"
        assert torch.equal(a, b), f"{tag}[{i}]: bits differ"


def _poisoned(tag, op, tail_bytes, shape, call):
    import learned_kv_block_amd as msa
    n = msa.workspace_size(shape, op)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ref = [t.clone() for t in call(ws)]
    pb = min(tail_bytes, n)
    for _ in range(2):
        ws.zero_()
        ws[n - pb:].fill_(255)
        got = call(ws)
        torch.cuda.synchronize()
        _same(tag, ref, got)
    print(f"[workspace] {tag}: {pb} of {n} bytes poisoned, outputs identical", flush=True)


def test_outputs_independent_of_workspace_contents():
    """Training workload (2 x 32768 tokens): selection (bf16 and FP8 index), attention
    backward and index backward."""
    import learned_kv_block_amd as msa
    cfg = si.CONFIGS["train_b2_n32768"]
    print(f"[workspace] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg, names=("q", "k", "v", "q_idx", "k_idx", "dout"))
    B, Hkv, K, D, DI = cfg.batch, cfg.num_kv_heads, cfg.topk, cfg.head_dim, cfg.idx_dim
    sh = msa.make_shape(B, cfg.seqlen_kv, cfg.seqlen_q, 0, cfg.num_q_heads, Hkv, D, DI, K,
                        msa.MSA_BF16)
    _poisoned("select", msa.MSA_OP_SELECT, 1 << 40, sh,
              lambda ws: (lambda r: (r["ids"], r["margin"]))(
                  msa.msa_select(x["q_idx"], x["k_idx"], K, want_margin=True,
                                 num_q_heads=cfg.num_q_heads, head_dim=D, workspace=ws)))
    qz = msa.msa_index_quantize_fp8(x["q_idx"], x["k_idx"], num_q_heads=cfg.num_q_heads,
                                    head_dim=D)
    _poisoned("select_fp8", msa.MSA_OP_SELECT, 1 << 40, sh,
              lambda ws: (lambda r: (r["ids"], r["margin"]))(
                  msa.msa_select_fp8(qz["q8"], qz["q_exp"], qz["k8"], qz["k_exp"], K,
                                     want_margin=True, num_q_heads=cfg.num_q_heads, head_dim=D,
                                     workspace=ws)))
    del qz
    ids = msa.msa_select(x["q_idx"], x["k_idx"], K, num_q_heads=cfg.num_q_heads,
                         head_dim=D)["ids"]
    out, lse = msa.msa_attn_fwd(x["q"], x["k"], x["v"], ids, idx_dim=DI)
    slabs = B * Hkv * cfg.num_blocks + 2 * 512
    _poisoned("attn_bwd", msa.MSA_OP_ATTN_BWD, slabs * 2 * 2 * 128 * D * 4, sh,
              lambda ws: msa.msa_attn_bwd(x["q"], x["k"], x["v"], ids, out, lse, x["dout"],
                                          idx_dim=DI, workspace=ws))
    kl = msa.msa_kl_align(x["q"], x["k"], x["q_idx"], x["k_idx"], ids, lse)
    _poisoned("idx_bwd", msa.MSA_OP_IDX_BWD, slabs * 128 * DI * 4, sh,
              lambda ws: msa.msa_idx_bwd(x["q_idx"], x["k_idx"], ids, kl["dlogits"], 1.0,
                                         num_q_heads=cfg.num_q_heads, head_dim=D, workspace=ws))


def test_dense_kl_bwd_independent_of_workspace_contents():
    """Warm-up stage, 2 x 32768 tokens: msa_kl_dense_bwd's workspace holds only bf16 dS values
    and fp32 dk_idx accumulators, so all of it is filled."""
    import learned_kv_block_amd as msa
    cfg = si.CONFIGS["train_b2_n32768"]
    print(f"[workspace] start dense {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg, names=("q", "k", "q_idx", "k_idx"))
    lse_main = msa.msa_dense_lse(x["q"], x["k"], idx_dim=cfg.idx_dim)
    sh = msa.make_shape(cfg.batch, cfg.seqlen_kv, cfg.seqlen_q, 0, cfg.num_q_heads,
                        cfg.num_kv_heads, cfg.head_dim, cfg.idx_dim, 1, msa.MSA_BF16)
    keys = ("lse_idx", "dq_idx", "dk_idx", "kl_rows", "kl_mean", "block_mass")
    _poisoned("kl_dense_bwd", msa.MSA_OP_KL_DENSE_BWD, 1 << 40, sh,
              lambda ws: (lambda r: [r[k] for k in keys])(
                  msa.msa_kl_dense_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], lse_main, 0.5,
                                       want_mass=True, workspace=ws)))
