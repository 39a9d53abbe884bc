"""Block selection with exact score ties, on the GPU through the C ABI.

The sampled parity tests exempt rows whose k-th and (k+1)-th block scores are
closer than 1e-4, so they cannot see the tie rule. Here the block scores are
small integers over sqrt(d_idx) = 8, exact in fp32 and fp64 alike, so the
selection is fixed by the rule itself: larger score first, the lower block
index among equal scores, selected blocks in ascending order, the local block
floor(i/128) last (block-selection and selector-supervision passages: a
softmax-free Top-k with a fixed secondary key). The expected ids follow from
the construction in closed form; every row must match exactly.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

N = 20000          # 157 blocks: local blocks up to 156, past the 128 candidates ranked in LDS
HKV, G, D_IDX, TOPK = 2, 2, 64, 16


def _expected(block_vals, n_rows):
    """ids [n_rows, TOPK] for scores block_vals[b] (identical for every row)."""
    out = np.full((n_rows, TOPK), -1, dtype=np.int32)
    for i in range(n_rows):
        L = i // 128
        if L + 1 <= TOPK:
            out[i, :L + 1] = np.arange(L + 1)
            continue
        cand = np.arange(L)
        order = np.lexsort((cand, -block_vals[:L]))  # score desc, then block asc
        sel = np.sort(cand[order[:TOPK - 1]])
        out[i, :TOPK - 1] = sel
        out[i, TOPK - 1] = L
    return out


def _run(q_idx, k_idx):
    import learned_kv_block_amd as msa
    res = msa.msa_select(q_idx, k_idx, TOPK, want_margin=True, num_q_heads=HKV * G, head_dim=64)
    torch.cuda.synchronize()
    return res["ids"].cpu().numpy(), res["margin"].cpu().numpy()


def test_all_scores_equal():
    # every block score is 0: the lowest indices win; rows with more than 128
    # tied candidates take the argmax fallback
    dev = torch.device("cuda:0")
    q_idx = torch.zeros((1, N, HKV, D_IDX), dtype=torch.bfloat16, device=dev)
    g = torch.Generator().manual_seed(5)
    k_idx = torch.randn((1, N, D_IDX), generator=g).to(torch.bfloat16).to(dev)
    ids, margin = _run(q_idx, k_idx)
    exp = _expected(np.zeros(N // 128 + 1), N)
    for r in range(HKV):
        np.testing.assert_array_equal(ids[0, :, r], exp)
    L = np.arange(N) // 128
    m = margin[0]
    assert np.all(m[L + 1 <= TOPK] == np.inf)
    assert np.all(m[L + 1 > TOPK] == 0.0)


def test_few_distinct_scores():
    # block b scores v_b / 8 with v_b in 1..6: long runs of equal scores around
    # the cut-off
    dev = torch.device("cuda:0")
    nb = (N + 127) // 128
    rng = np.random.default_rng(17)
    v = rng.integers(1, 7, size=nb)
    kk = np.zeros((N, D_IDX), dtype=np.float32)
    for j in range(N):
        kk[j, :v[j // 128]] = 1.0
    q_idx = torch.ones((1, N, HKV, D_IDX), dtype=torch.bfloat16, device=dev)
    k_idx = torch.from_numpy(kk).to(torch.bfloat16).unsqueeze(0).to(dev)
    ids, margin = _run(q_idx, k_idx)
    exp = _expected(v.astype(np.float64), N)
    for r in range(HKV):
        np.testing.assert_array_equal(ids[0, :, r], exp)
    # margin: worst selected minus best unselected score, exact (+inf when
    # every visible block is selected)
    assert np.all(margin[0, :TOPK * 128] == np.inf)
    for i in (TOPK * 128, 5000, N - 1):
        L = i // 128
        sel = exp[i, :TOPK - 1]
        rest = np.setdiff1d(np.arange(L), sel)
        want = (v[sel].min() - v[rest].max()) / 8.0
        for r in range(HKV):
            assert margin[0, i, r] == np.float32(want), (i, r, margin[0, i, r], want)
