"""bf16 rows whose two competing blocks differ below fp32 resolution: the near-tie rule.

Parity compares block ids bit for bit except in rows whose oracle cutoff margin (the
selector-supervision page's eq. 9: score of the last block taken minus score of the
best block left out) is below 1e-4; such a row may pick either block but must still be
a valid selection within 1e-4 of the oracle's cutoff, and its outputs are compared on
the GPU's own ids. Random inputs rarely produce such rows, so here they are built:

  q_idx = (1, 2^-10, 0, ...) for every row; in K_idx, blocks 1 and 4 hold a token
  with component 0 = 2^21 (clear winners), block 2 a token (2^20, 0, ...) and block 5
  a token (2^20, 2^-4, ...); every other token is small.

In exact arithmetic block 5 outscores block 2 by 2^-14 / sqrt(64): the oracle (fp64)
takes {1, 4, 5} and the local block. In fp32 the sum 2^20 + 2^-14 rounds to 2^20 (the
fp32 spacing at 2^20 is 2^-3), the two blocks tie, and the lower index wins: the GPU
takes {1, 2, 4}. Every row of the last query block is such a near tie, so the validity
branch of the id check runs on bf16 ids, and out / LSE are checked on the GPU's ids.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import parity

pytestmark = pytest.mark.gpu

N, HKV, G, D, D_IDX, TOPK = 1024, 2, 8, 128, 64, 4


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_bf16_near_tie_rows_take_the_validity_branch():
    import learned_kv_block_amd as msa
    dev = torch.device("cuda:0")
    q_start, Nq = 7 * 128, 128  # queries in the last block: local block 7, candidates 0..6
    g = torch.Generator().manual_seed(31)
    kk = (torch.rand((N, D_IDX), generator=g) - 0.5)  # |k| < 0.5: far below the planted tokens
    for blk, val in ((1, 2.0 ** 21), (4, 2.0 ** 21), (2, 2.0 ** 20), (5, 2.0 ** 20)):
        kk[blk * 128 + 17] = 0.0
        kk[blk * 128 + 17, 0] = val
    kk[5 * 128 + 17, 1] = 2.0 ** -4
    k_idx = kk.to(torch.bfloat16).unsqueeze(0).to(dev)
    qi = torch.zeros((1, Nq, HKV, D_IDX))
    qi[..., 0] = 1.0
    qi[..., 1] = 2.0 ** -10
    q_idx = qi.to(torch.bfloat16).to(dev)
    q = (torch.randn((1, Nq, HKV * G, D), generator=g) * 0.7).to(torch.bfloat16).to(dev)
    k = (torch.randn((1, N, HKV, D), generator=g) * 0.7).to(torch.bfloat16).to(dev)
    v = (torch.randn((1, N, HKV, D), generator=g) * 0.7).to(torch.bfloat16).to(dev)

    sel = msa.msa_select(q_idx, k_idx, TOPK, q_start=q_start, want_scores=True, want_margin=True,
                         num_q_heads=HKV * G, head_dim=D)
    out, lse = msa.msa_attn_fwd(q, k, v, sel["ids"], q_start=q_start, idx_dim=D_IDX)
    torch.cuda.synchronize()
    gids = sel["ids"][0].cpu().numpy()
    assert np.all(gids == np.array([1, 2, 4, 7], dtype=np.int32)), "the fp32 tie must pick block 2"

    shp = oracle.RefShape(1, N, Nq, q_start, HKV * G, HKV, D, D_IDX, 128, TOPK, 1)
    ref = oracle.select(shp, _bits(q_idx[0]), _bits(k_idx), want_scores=True, want_margin=True)
    assert np.all(ref["ids"] == np.array([1, 4, 5, 7], dtype=np.int32))
    assert np.all(ref["margin"] > 0) and np.all(ref["margin"] < parity.NEAR_TIE)
    report = {}
    near = parity.check_ids(parity.si.CONFIGS["main_n8192"], gids, ref, report)
    assert near == Nq * HKV  # every row is a near tie, and every one passed the validity check
    # the GPU's scores: the tied blocks both score 2^20 / 8 exactly
    sc = sel["block_scores"][0].cpu().numpy()
    assert np.all(sc[:, :, 2] == sc[:, :, 5])
    # outputs on the GPU's own ids
    o_ref, l_ref = oracle.attn(shp, _bits(q[0]), _bits(k), _bits(v), gids)
    t = dict(max_abs=1e-2, rel_l2=5e-3)
    parity.check_close("out", out[0].float().cpu().numpy(), o_ref, t, report)
    parity.check_close("lse", lse[0].cpu().numpy(), l_ref, t, report)
    print("[near-tie]", report)
