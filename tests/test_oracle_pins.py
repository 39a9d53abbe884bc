"""Pins of the fp64 oracle against facts outside the oracle itself.

Each test names the passage or the mathematical fact it checks. Mistakes these
catch: a dropped causal mask, a wrong scale, a swapped KL direction, a logit
(instead of probability) average in the teacher, a wrong tie rule, an
off-by-one in the local block, a transposed operand, a wrong slot mapping.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import diagnostics as dg

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def shape(**kw):
    base = dict(batch=1, seqlen_kv=256, seqlen_q=256, q_start=0, num_q_heads=4, num_kv_heads=2,
                head_dim=16, idx_dim=8, block_size=32, topk=3, dtype=0)
    base.update(kw)
    return oracle.RefShape(*[base[f] for f, _ in oracle.RefShape._fields_])


def rnd(rng, *shp, scale=1.0):
    return (rng.standard_normal(shp) * scale).astype(np.float32)


# ----------------------------------------------------------------------- worked examples


def test_superv_fig1_worked_example_selection():
    """"4.1.1 · 监督与联合训练" Fig. 1: student scores (0.7, -0.2, 1.1), k=2 select positions
    {1, 3} (1-based); against teacher (0.50, 0.30, 0.20) recall 1/2, coverage 0.70.

    Built end to end: three 128-token blocks, d_idx=1, q_idx=1 so the index logit of a token
    is its K_idx value; the query is the last token, so block 2 is its local block."""
    g = json.load(open(os.path.join(GOLD, "superv_worked_examples.json")))["figure1"]
    Bk, nb = 128, 3
    k_idx = np.full((1, nb * Bk, 1), -5.0, dtype=np.float32)
    for b, sc in enumerate(g["student_scores"]):
        k_idx[0, b * Bk + 17, 0] = sc
    q_idx = np.ones((1, 1, 1), dtype=np.float32)
    sh = shape(seqlen_kv=nb * Bk, seqlen_q=1, q_start=nb * Bk - 1, num_q_heads=1, num_kv_heads=1,
               idx_dim=1, block_size=Bk, topk=g["k"])
    out = oracle.select(sh, q_idx, k_idx, want_scores=True, want_margin=True)
    assert out["ids"][0, 0].tolist() == g["selected"]
    np.testing.assert_allclose(out["block_scores"][0, 0],
                               np.float32(g["student_scores"]).astype(np.float64))
    assert dg.teacher_topk(np.array(g["teacher"]), g["k"]).tolist() == g["teacher_topk"]
    assert dg.set_recall(out["ids"][0, 0], np.array(g["teacher"]), g["k"]) == g["recall"]
    assert math.isclose(dg.coverage(out["ids"][0, 0], np.array(g["teacher"])), g["coverage"])


def test_superv_recall_coverage_examples():
    """"4.1.1" eq. (2)(3) example and the 8-block budget example."""
    g = json.load(open(os.path.join(GOLD, "superv_worked_examples.json")))
    ex = g["eq2_eq3_example"]
    p = np.array(ex["teacher"])
    for c in ex["candidates"]:
        assert dg.set_recall(c["selected"], p, ex["k"]) == c["recall"]
        assert math.isclose(dg.coverage(c["selected"], p), c["coverage"], abs_tol=1e-12)
    bx = g["budget_example"]
    p = np.array(bx["teacher"])
    assert math.isclose(dg.coverage(dg.teacher_topk(p, bx["k"]), p), bx["oracle_coverage"],
                        abs_tol=1e-12)
    assert math.isclose(dg.set_recall(bx["selected"], p, bx["k"]), bx["recall"])
    assert math.isclose(dg.coverage(bx["selected"], p), bx["coverage"], abs_tol=1e-12)


def test_relative_output_error_definition():
    """"4.1.1" eq. (14) on a hand example: ||(3,4)-(0,0)|| / ||(0,0)+..|| style values."""
    assert math.isclose(dg.relative_output_error([1.0, 2.0], [1.0, 2.0]), 0.0)
    assert math.isclose(dg.relative_output_error([3.0, 0.0], [0.0, 4.0]), 5.0 / 4.0, rel_tol=1e-9)


def test_native_two_token_example():
    """"2.4 · 训练原生稀疏" hand calculation: weights (0.75, 0.25) on v1=(2,0), v2=(0,2) give
    o=(1.5, 0.5). Logits (ln 3, 0) give those weights; LSE = ln(3+1)."""
    g = json.load(open(os.path.join(GOLD, "native_two_token_example.json")))
    d = 2
    sh = shape(seqlen_kv=2, seqlen_q=1, q_start=1, num_q_heads=1, num_kv_heads=1, head_dim=d,
               idx_dim=1, block_size=128, topk=1)
    # q . k / sqrt(2): q = (sqrt(2) ln3, 0), k1 = (1, 0), k2 = (0, 0)
    q = np.array([[[math.sqrt(2.0) * g["logits"][0], 0.0]]], dtype=np.float32)
    k = np.array([[[[1.0, 0.0]], [[0.0, 0.0]]]], dtype=np.float32)
    v = np.array([[[g["values"][0]], [g["values"][1]]]], dtype=np.float32)
    ids = np.zeros((1, 1, 1), dtype=np.int32)
    o, lse = oracle.attn(sh, q, k, v, ids)
    # q is rounded to fp32, so the logit is ln3 to ~1e-7
    np.testing.assert_allclose(o[0, 0], g["output"], atol=1e-6)
    assert abs(lse[0, 0] - g["lse"]) < 1e-6


# ----------------------------------------------------------------------- selection rule


def test_topk_brute_force_over_subsets():
    """With distinct scores, the k-1 non-local blocks chosen are the (k-1)-subset of blocks
    0..L-1 with the largest score sum (brute force over all subsets); the local block L is
    always in the list; ids ascending."""
    rng = np.random.default_rng(0)
    for _ in range(200):
        L = int(rng.integers(0, 10))
        k = int(rng.integers(1, 6))
        M = rng.standard_normal(L + 1)
        ids, _ = oracle.topk_row(M, L, k)
        if L + 1 <= k:
            assert ids.tolist() == list(range(L + 1)) + [-1] * (k - L - 1)
            continue
        best = max(itertools.combinations(range(L), k - 1), key=lambda c: sum(M[list(c)]))
        assert ids.tolist() == sorted(best) + [L]


def test_topk_exact_ties_prefer_lower_index():
    """Tie rule ("4.1.1" §1.2: ties at the cutoff need a fixed secondary key): equal block
    scores rank the lower block index first."""
    M = [1.0, 3.0, 3.0, 2.0, 3.0, 0.5]
    ids, mg = oracle.topk_row(M, 5, 3)
    assert ids.tolist() == [1, 2, 5]
    assert mg == 0.0
    ids, _ = oracle.topk_row([0.0, 0.0, 0.0, 0.0, 0.0], 4, 3)
    assert ids.tolist() == [0, 1, 4]


def test_topk_forced_local_block_and_short_rows():
    """The local block is kept even with the lowest score ("MSA Indexer vs DSA" §2.2; blog);
    rows with fewer than k visible blocks select all of them and pad with -1."""
    ids, _ = oracle.topk_row([5.0, 4.0, 3.0, -100.0], 3, 2)
    assert ids.tolist() == [0, 3]
    ids, mg = oracle.topk_row([0.1, 0.2], 1, 4)
    assert ids.tolist() == [0, 1, -1, -1] and math.isinf(mg)


def test_topk_margin():
    """Cutoff margin ("4.1.1" eq. 9): last taken score minus best left-out score."""
    ids, mg = oracle.topk_row([1.0, 0.5, 0.7, 0.2, -3.0], 4, 3)
    assert ids.tolist() == [0, 2, 4]
    assert math.isclose(mg, 0.2, abs_tol=1e-15)


def test_topk_on_raw_scores_equals_topk_on_softmax():
    """Blog, kernel lessons: softmax preserves order, so Top-k on raw scores equals Top-k on
    their softmax (fp64, well-separated random rows)."""
    rng = np.random.default_rng(1)
    for _ in range(100):
        L = int(rng.integers(1, 60))
        M = rng.standard_normal(L + 1)
        e = np.exp(M - M.max())
        P = e / e.sum()
        assert oracle.topk_row(M, L, 7)[0].tolist() == oracle.topk_row(P, L, 7)[0].tolist()


# ----------------------------------------------------------------------- index logits / block max


@pytest.mark.parametrize("N,Bk,q_start,Nq", [(200, 32, 0, 200), (300, 64, 120, 100)])
def test_block_scores_match_masked_matmul(N, Bk, q_start, Nq):
    """"MSA Indexer vs DSA" §2.1-§2.2: S_idx = Q_idx K_idx^T / sqrt(d_idx) with one shared K_idx
    head; block score = max over j in the block with j <= i. Checked against a library matmul
    of the whole N x N matrix, masked and reshaped to blocks; the block LSE ("KL alignment"
    §6) against a library logsumexp of the same masked blocks."""
    rng = np.random.default_rng(2)
    B, H, di, k = 2, 3, 8, 2
    sh = shape(batch=B, seqlen_kv=N, seqlen_q=Nq, q_start=q_start, num_q_heads=H,
               num_kv_heads=H, idx_dim=di, block_size=Bk, topk=k)
    q_idx = rnd(rng, B, Nq, H, di)
    k_idx = rnd(rng, B, N, di)
    out = oracle.select(sh, q_idx.reshape(B * Nq, H, di), k_idx, want_scores=True, want_lse=True)
    nb = (N + Bk - 1) // Bk
    from scipy.special import logsumexp
    for b in range(B):
        S = np.einsum("thc,jc->thj", q_idx[b].astype(np.float64), k_idx[b].astype(np.float64))
        S /= math.sqrt(di)
        for t in range(Nq):
            i = q_start + t
            for h in range(H):
                for blk in range(nb):
                    got = out["block_scores"][b * Nq + t, h, blk]
                    gl = out["block_lse"][b * Nq + t, h, blk]
                    seg = S[t, h, blk * Bk:min(blk * Bk + Bk, i + 1)]
                    if blk * Bk > i:
                        assert got == -np.inf and gl == -np.inf
                    else:
                        assert abs(got - seg.max()) < 1e-12
                        assert abs(gl - logsumexp(seg)) < 1e-12


def test_row_subset_equals_full_run():
    """Rows are independent: evaluating a subset of rows gives the same rows as a full run."""
    rng = np.random.default_rng(3)
    sh = shape(seqlen_kv=200, seqlen_q=200)
    q_idx = rnd(rng, 200, 2, 8)
    k_idx = rnd(rng, 1, 200, 8)
    full = oracle.select(sh, q_idx, k_idx)["ids"]
    rows = np.array([0, 31, 32, 150, 199])
    sub = oracle.select(sh, q_idx[rows], k_idx, rows=rows)["ids"]
    np.testing.assert_array_equal(sub, full[rows])


# ----------------------------------------------------------------------- attention


def _dense_sdpa(q, k, v, G, q_start):
    """Library causal SDPA in fp64 on CPU; GQA by repeating KV heads (group of head h = h//G)."""
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)  # B,Hq,Nq,d
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    Nq, N = qt.shape[2], kt.shape[2]
    i = torch.arange(Nq)[:, None] + q_start
    j = torch.arange(N)[None, :]
    mask = j <= i
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    s = (qt @ kt.transpose(-1, -2)) / math.sqrt(q.shape[-1])
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


@pytest.mark.parametrize("N,Nq,q_start,Bk", [(300, 300, 0, 64), (257, 100, 157, 32)])
def test_k_all_blocks_is_dense_causal_attention(N, Nq, q_start, Bk):
    """"2.4 · 训练原生稀疏": with k covering every block, block-sparse attention with the current
    block forced is full causal attention. Checked end to end (select -> attn) against the
    library's causal scaled_dot_product_attention in fp64, GQA with G=2, ragged last block."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, d, di = 2, 4, 2, 16, 8
    nb = (N + Bk - 1) // Bk
    sh = shape(batch=B, seqlen_kv=N, seqlen_q=Nq, q_start=q_start, num_q_heads=Hq,
               num_kv_heads=Hkv, head_dim=d, idx_dim=di, block_size=Bk, topk=nb)
    q = rnd(rng, B, Nq, Hq, d)
    k = rnd(rng, B, N, Hkv, d)
    v = rnd(rng, B, N, Hkv, d)
    q_idx = rnd(rng, B * Nq, Hkv, di)
    k_idx = rnd(rng, B, N, di)
    ids = oracle.select(sh, q_idx, k_idx)["ids"]
    for row in range(B * Nq):
        L = (q_start + row % Nq) // Bk
        for r in range(Hkv):
            assert ids[row, r].tolist() == list(range(L + 1)) + [-1] * (nb - L - 1)
    o, lse = oracle.attn(sh, q.reshape(B * Nq, Hq, d), k, v, ids)
    o_ref, lse_ref = _dense_sdpa(q, k, v, Hq // Hkv, q_start)
    np.testing.assert_allclose(o.reshape(B, Nq, Hq, d), o_ref, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse.reshape(B, Nq, Hq), lse_ref, atol=1e-12, rtol=1e-12)


def test_sparse_attention_is_restricted_softmax_on_explicit_mask():
    """"2.4 · 训练原生稀疏" eq. (2): softmax with the denominator restricted to the selected
    set. The mask is built here from the ids (token j allowed iff its block is listed and
    j <= i) and applied to library softmax; query head h reads KV head h // G."""
    rng = np.random.default_rng(5)
    B, N, Hq, Hkv, d, di, Bk, k = 1, 256, 4, 2, 16, 8, 32, 3
    sh = shape(batch=B, seqlen_kv=N, seqlen_q=N, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
               idx_dim=di, block_size=Bk, topk=k)
    q = rnd(rng, N, Hq, d)
    kk = rnd(rng, 1, N, Hkv, d)
    v = rnd(rng, 1, N, Hkv, d)
    ids = oracle.select(sh, rnd(rng, N, Hkv, di), rnd(rng, 1, N, di))["ids"]
    o, lse = oracle.attn(sh, q, kk, v, ids)
    G = Hq // Hkv
    for t in range(0, N, 7):
        for h in range(Hq):
            r = h // G
            allowed = np.array([(j // Bk) in ids[t, r].tolist() and j <= t for j in range(N)])
            s = torch.from_numpy(kk[0, :, r].astype(np.float64)) @ torch.from_numpy(
                q[t, h].astype(np.float64)) / math.sqrt(d)
            s[~torch.from_numpy(allowed)] = float("-inf")
            w = torch.softmax(s, dim=0)
            ref = w @ torch.from_numpy(v[0, :, r].astype(np.float64))
            np.testing.assert_allclose(o[t, h], ref.numpy(), atol=1e-12)
            assert abs(lse[t, h] - torch.logsumexp(s, 0).item()) < 1e-12


def test_decode_row_equals_prefill_row():
    """"2.4 · 训练原生稀疏" §1.2: prefill and decode must share the math. A single query at
    position N-1 (decode) gives the same ids, output and LSE as the last row of prefill."""
    rng = np.random.default_rng(6)
    N, Hq, Hkv, d, di, Bk, k = 320, 4, 2, 16, 8, 32, 4
    full = shape(seqlen_kv=N, seqlen_q=N, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                 idx_dim=di, block_size=Bk, topk=k)
    dec = shape(seqlen_kv=N, seqlen_q=1, q_start=N - 1, num_q_heads=Hq, num_kv_heads=Hkv,
                head_dim=d, idx_dim=di, block_size=Bk, topk=k)
    q, q_idx = rnd(rng, N, Hq, d), rnd(rng, N, Hkv, di)
    kk, v, k_idx = rnd(rng, 1, N, Hkv, d), rnd(rng, 1, N, Hkv, d), rnd(rng, 1, N, di)
    ids_f = oracle.select(full, q_idx, k_idx)["ids"]
    ids_d = oracle.select(dec, q_idx[-1:], k_idx)["ids"]
    np.testing.assert_array_equal(ids_d[0], ids_f[-1])
    o_f, l_f = oracle.attn(full, q, kk, v, ids_f)
    o_d, l_d = oracle.attn(dec, q[-1:], kk, v, ids_d)
    np.testing.assert_array_equal(o_d[0], o_f[-1])
    np.testing.assert_array_equal(l_d[0], l_f[-1])


# ----------------------------------------------------------------------- KL alignment


def test_kl_gradient_is_finite_difference_of_kl():
    """"KL alignment" §3: d KL(P || P_idx) / d z_j = P_idx_j - P_j with the teacher detached.
    Central differences (h = 1e-6) of the oracle's own KL value in the index logits."""
    rng = np.random.default_rng(7)
    for G, n in [(1, 5), (4, 37), (16, 130)]:
        sm = rng.standard_normal((G, n)) * 2
        si = rng.standard_normal(n) * 2
        base = oracle.kl_row(sm, si)
        h = 1e-6
        for j in rng.choice(n, size=min(n, 12), replace=False):
            sp, sn = si.copy(), si.copy()
            sp[j] += h
            sn[j] -= h
            fd = (oracle.kl_row(sm, sp)["kl"] - oracle.kl_row(sm, sn)["kl"]) / (2 * h)
            assert abs(fd - base["dS"][j]) < 1e-8, (G, n, j, fd, base["dS"][j])


def test_kl_probability_average_hand_example():
    """"KL alignment" §2.2: the teacher averages the heads' probabilities, not their logits.
    Heads with logits (0, ln 3) and (0, 0) give probabilities (1/4, 3/4) and (1/2, 1/2), so
    P = (3/8, 5/8) (a logit average would give softmax(0, ln(3)/2) = (0.366.., 0.633..)).
    Student logits (0, 0) give P_idx = (1/2, 1/2): KL = 3/8 ln(3/4) + 5/8 ln(5/4),
    gradient P_idx - P = (1/8, -1/8)."""
    out = oracle.kl_row([[0.0, math.log(3.0)], [0.0, 0.0]], [0.0, 0.0])
    np.testing.assert_allclose(out["P"], [3 / 8, 5 / 8], atol=1e-15)
    np.testing.assert_allclose(out["P_idx"], [0.5, 0.5], atol=1e-15)
    assert abs(out["kl"] - (3 / 8 * math.log(3 / 4) + 5 / 8 * math.log(5 / 4))) < 1e-15
    np.testing.assert_allclose(out["dS"], [1 / 8, -1 / 8], atol=1e-15)


def test_kl_invariants():
    """KL >= 0; gradient sums to 0 (both distributions sum to 1); KL = CE - H ("KL alignment"
    §3, soft-label cross entropy minus the teacher entropy); equal distributions give 0."""
    rng = np.random.default_rng(8)
    for _ in range(50):
        G, n = int(rng.integers(1, 8)), int(rng.integers(1, 200))
        sm = rng.standard_normal((G, n)) * 3
        si = rng.standard_normal(n) * 3
        o = oracle.kl_row(sm, si)
        assert o["kl"] >= -1e-15
        assert abs(o["dS"].sum()) < 1e-12
        ce = -np.sum(o["P"] * np.log(o["P_idx"]))
        H = -np.sum(o["P"] * np.log(o["P"]))
        assert abs(o["kl"] - (ce - H)) < 1e-10
    sm = rng.standard_normal((1, 9))
    o = oracle.kl_row(sm, sm[0])
    assert abs(o["kl"]) < 1e-15 and np.abs(o["dS"]).max() < 1e-15


def test_kl_identical_branches_and_first_row():
    """End to end: with G=1, Hkv=1, d_idx=d and Q_idx=Q, K_idx=K the index branch equals the
    teacher, so KL = 0 and dS = 0 on every row. Row i=0 has a one-token support: KL = 0."""
    rng = np.random.default_rng(9)
    N, d, Bk, k = 160, 16, 32, 3
    sh = shape(seqlen_kv=N, seqlen_q=N, num_q_heads=1, num_kv_heads=1, head_dim=d, idx_dim=d,
               block_size=Bk, topk=k)
    q = rnd(rng, N, 1, d)
    kk = rnd(rng, 1, N, 1, d)
    ids = oracle.select(sh, q, kk[:, :, 0, :])["ids"]
    out = oracle.kl(sh, q, kk, q, kk[:, :, 0, :], ids)
    assert np.abs(out["kl_rows"]).max() < 1e-12
    assert np.abs(out["dlogits"]).max() < 1e-12
    sh2 = shape(seqlen_kv=N, seqlen_q=N, head_dim=d, idx_dim=8, block_size=Bk, topk=k)
    q2, qi2 = rnd(rng, N, 4, d), rnd(rng, N, 2, 8)
    kk2, ki2 = rnd(rng, 1, N, 2, d), rnd(rng, 1, N, 8)
    ids2 = oracle.select(sh2, qi2, ki2)["ids"]
    o2 = oracle.kl(sh2, q2, kk2, qi2, ki2, ids2)
    assert np.abs(o2["kl_rows"][0]).max() < 1e-15
    assert np.abs(o2["dlogits"][0]).max() < 1e-15


def test_kl_dense_support_matches_full_context_logits():
    """"KL alignment" §5 (warm-up): with k covering every block the support is the full causal
    context. The row KL and its gradient then equal kl_row on logits built here by library
    matmuls over j <= i; the slot layout puts token j at (j // Bk, j % Bk). Also checks the
    two routes to LSE_idx ("KL alignment" §6): logsumexp over J equals the logsumexp of the
    per-block LSEs of the selected blocks."""
    rng = np.random.default_rng(10)
    N, Hq, Hkv, d, di, Bk = 100, 4, 2, 16, 8, 32
    nb = (N + Bk - 1) // Bk
    sh = shape(seqlen_kv=N, seqlen_q=N, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
               idx_dim=di, block_size=Bk, topk=nb)
    q, qi = rnd(rng, N, Hq, d), rnd(rng, N, Hkv, di)
    kk, ki = rnd(rng, 1, N, Hkv, d), rnd(rng, 1, N, di)
    sel = oracle.select(sh, qi, ki, want_lse=True)
    out = oracle.kl(sh, q, kk, qi, ki, sel["ids"])
    G = Hq // Hkv
    from scipy.special import logsumexp
    for t in [0, 1, 31, 32, 70, 99]:
        for r in range(Hkv):
            K = kk[0, :t + 1, r].astype(np.float64)
            sm = np.stack([K @ q[t, r * G + h].astype(np.float64) / math.sqrt(d)
                           for h in range(G)])
            si = ki[0, :t + 1].astype(np.float64) @ qi[t, r].astype(np.float64) / math.sqrt(di)
            ref = oracle.kl_row(sm, si)
            assert abs(out["kl_rows"][t, r] - ref["kl"]) < 1e-12
            dl = out["dlogits"][t, r].reshape(-1)[:t + 1]
            np.testing.assert_allclose(dl, ref["dS"], atol=1e-14)
            assert np.all(out["dlogits"][t, r].reshape(-1)[t + 1:] == 0.0)
            L = t // Bk
            two = logsumexp(sel["block_lse"][t, r, :L + 1])
            assert abs(two - out["lse_idx"][t, r]) < 1e-12
    assert abs(out["kl_mean"] - out["kl_rows"].mean()) < 1e-15


# ----------------------------------------------------------------------- backward


def test_dense_ids_are_the_k_all_selection():
    """dense_ids (the warm-up support, "KL alignment" §5) equals what the selection returns when
    k covers every block: blocks 0..floor(i/Bk) in order, then -1."""
    rng = np.random.default_rng(21)
    N, Nq, q_start, Bk = 300, 120, 180, 64
    nb = (N + Bk - 1) // Bk
    sh = shape(batch=2, seqlen_kv=N, seqlen_q=Nq, q_start=q_start, block_size=Bk, topk=nb)
    ids = oracle.select(sh, rnd(rng, 2 * Nq, 2, 8), rnd(rng, 2, N, 8))["ids"]
    np.testing.assert_array_equal(oracle.dense_ids(sh), ids)
    assert oracle.dense_shape(shape(seqlen_kv=N, block_size=Bk, topk=2)).topk == nb


def test_dense_block_mass_uniform_keys_closed_form():
    """Identical keys make every main logit of a head equal, so each head's softmax over the
    full causal context is uniform: P_j = 1/(i+1) and the mass of block b is (number of tokens
    j <= i in b)/(i+1). Ragged last block; G = 2 heads per group."""
    rng = np.random.default_rng(22)
    N, Bk, Hq, Hkv, d, di = 200, 32, 4, 2, 16, 8
    sh = oracle.dense_shape(shape(seqlen_kv=N, seqlen_q=N, num_q_heads=Hq, num_kv_heads=Hkv,
                                  head_dim=d, idx_dim=di, block_size=Bk))
    q = rnd(rng, N, Hq, d)
    kk = np.broadcast_to(rnd(rng, 1, 1, Hkv, d), (1, N, Hkv, d)).copy()
    out = oracle.kl(sh, q, kk, rnd(rng, N, Hkv, di), rnd(rng, 1, N, di), oracle.dense_ids(sh),
                    want_dlogits=False, want_mass=True)
    for t in [0, 5, 31, 32, 100, 199]:
        want = np.array([max(0, min(Bk, t + 1 - b * Bk)) for b in range(sh.topk)]) / (t + 1)
        for r in range(Hkv):
            np.testing.assert_allclose(out["block_mass"][t, r], want, atol=1e-14)


def test_dense_block_mass_is_library_softmax_mass():
    """"KL alignment" §2.2 and §8: the teacher is the mean over the group's heads of each head's
    softmax (probabilities averaged), and the block mass sums it over each block's tokens. Here
    the softmax is torch's over an explicit causal mask, the head mean and the block sums are
    numpy; the masses of every row sum to 1."""
    rng = np.random.default_rng(23)
    B, N, Nq, q_start, Bk, Hq, Hkv, d, di = 2, 150, 70, 80, 32, 8, 2, 16, 8
    sh = oracle.dense_shape(shape(batch=B, seqlen_kv=N, seqlen_q=Nq, q_start=q_start,
                                  num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, idx_dim=di,
                                  block_size=Bk))
    q = rnd(rng, B, Nq, Hq, d)
    kk = rnd(rng, B, N, Hkv, d)
    out = oracle.kl(sh, q.reshape(B * Nq, Hq, d), kk, rnd(rng, B * Nq, Hkv, di),
                    rnd(rng, B, N, di), oracle.dense_ids(sh), want_dlogits=False,
                    want_mass=True)
    G = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(kk.astype(np.float64))
    for b in range(B):
        s = torch.einsum("thd,jhd->thj", qt[b], kt[b].repeat_interleave(G, dim=1)) / math.sqrt(d)
        i = torch.arange(Nq)[:, None, None] + q_start
        s = s.masked_fill(torch.arange(N)[None, None, :] > i, float("-inf"))
        p = torch.softmax(s, dim=-1).numpy().reshape(Nq, Hkv, G, N).mean(axis=2)
        pad = np.zeros((Nq, Hkv, sh.topk * Bk))
        pad[..., :N] = p
        want = pad.reshape(Nq, Hkv, sh.topk, Bk).sum(axis=-1)
        got = out["block_mass"][b * Nq:(b + 1) * Nq]
        np.testing.assert_allclose(got, want, atol=1e-13)
        np.testing.assert_allclose(got.sum(axis=-1), 1.0, atol=1e-13)


def test_native_eq11_hand_gradient():
    """"2.4 · 训练原生稀疏" eq. (11) hand calculation: weights (0.75, 0.25), v1=(2,0), v2=(0,2),
    g=(1,-1) give logit gradients (0.75, -0.75). With z = q.k/sqrt(2), q = (sqrt(2) ln3, 0),
    k1 = (1, 0), k2 = (0, 0): dk_s = dz_s q/sqrt(2) = dz_s (ln3, 0), dv_s = alpha_s g,
    dq = sum_s dz_s k_s/sqrt(2)."""
    g = json.load(open(os.path.join(GOLD, "native_eq11_gradient_example.json")))
    d = 2
    sh = shape(seqlen_kv=2, seqlen_q=1, q_start=1, num_q_heads=1, num_kv_heads=1, head_dim=d,
               idx_dim=1, block_size=128, topk=1)
    q = np.array([[[math.sqrt(2.0) * g["logits"][0], 0.0]]], dtype=np.float32)
    k = np.array([[[[1.0, 0.0]], [[0.0, 0.0]]]], dtype=np.float32)
    v = np.array([[[g["values"][0]], [g["values"][1]]]], dtype=np.float32)
    dout = np.array([[g["upstream"]]], dtype=np.float32)
    ids = np.zeros((1, 1, 1), dtype=np.int32)
    dq, dk, dv = oracle.attn_bwd(sh, q, k, v, ids, dout)
    ln3 = float(q[0, 0, 0]) / math.sqrt(2.0)
    dz = [dk[0, 0, 0, 0] / ln3, dk[0, 1, 0, 0] / ln3]
    np.testing.assert_allclose(dz, g["logit_grad"], atol=1e-6)
    assert abs(dk[0, 0, 0, 1]) < 1e-12 and abs(dk[0, 1, 0, 1]) < 1e-12
    for s in range(2):
        np.testing.assert_allclose(dv[0, s, 0], np.array(g["upstream"]) * g["weights"][s], atol=1e-6)
    np.testing.assert_allclose(dq[0, 0], [g["logit_grad"][0] / math.sqrt(2.0), 0.0], atol=1e-6)


def _bwd_case(rng, B=1, N=200, Nq=200, q_start=0, Hq=4, Hkv=2, d=8, di=4, Bk=32, topk=3):
    sh = shape(batch=B, seqlen_kv=N, seqlen_q=Nq, q_start=q_start, num_q_heads=Hq,
               num_kv_heads=Hkv, head_dim=d, idx_dim=di, block_size=Bk, topk=topk)
    x = dict(q=rnd(rng, B * Nq, Hq, d), k=rnd(rng, B, N, Hkv, d), v=rnd(rng, B, N, Hkv, d),
             q_idx=rnd(rng, B * Nq, Hkv, di), k_idx=rnd(rng, B, N, di),
             dout=rnd(rng, B * Nq, Hq, d))
    x["ids"] = oracle.select(sh, x["q_idx"], x["k_idx"])["ids"]
    return sh, x


def test_attn_bwd_is_finite_difference_of_forward():
    """Gradients of L = sum(dout * O) with the selection held fixed ("2.4" eq. (12): the hard
    selection has zero derivative almost everywhere), by central differences of the oracle's
    own forward on fp32 inputs (the step is the fp32-rounded difference)."""
    rng = np.random.default_rng(21)
    sh, x = _bwd_case(rng, q_start=100, Nq=100, N=200)
    dq, dk, dv = oracle.attn_bwd(sh, x["q"], x["k"], x["v"], x["ids"], x["dout"])

    def loss(q, k, v):
        o, _ = oracle.attn(sh, q, k, v, x["ids"])
        return float(np.sum(o * x["dout"].astype(np.float64)))

    def fd(name, idx):
        a = x[name]
        p, m = a.copy(), a.copy()
        p[idx] = np.float32(a[idx] + np.float32(2e-3))
        m[idx] = np.float32(a[idx] - np.float32(2e-3))
        args = {n: x[n] for n in ("q", "k", "v")}
        lp = loss(**{**args, name: p})
        lm = loss(**{**args, name: m})
        return (lp - lm) / (float(p[idx]) - float(m[idx]))

    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        a = x[name]
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in a.shape)
            f = fd(name, idx)
            assert abs(f - grad[idx]) < 2e-5 * max(1.0, abs(f)), (name, idx, f, grad[idx])


def test_attn_bwd_k_all_blocks_is_dense_autograd():
    """With k covering every block the sparse attention is dense causal attention ("2.4"), so
    its gradients equal the library's autograd of causal scaled_dot_product_attention in fp64
    (GQA G=2, ragged last block, chunked queries)."""
    rng = np.random.default_rng(22)
    B, N, Nq, q_start, Hq, Hkv, d, Bk = 2, 150, 60, 90, 4, 2, 8, 32
    nb = (N + Bk - 1) // Bk
    sh, x = _bwd_case(rng, B=B, N=N, Nq=Nq, q_start=q_start, Hq=Hq, Hkv=Hkv, d=d, Bk=Bk, topk=nb)
    dq, dk, dv = oracle.attn_bwd(sh, x["q"], x["k"], x["v"], x["ids"], x["dout"])
    G = Hq // Hkv
    qt = torch.tensor(x["q"].reshape(B, Nq, Hq, d), dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(x["k"], dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(x["v"], dtype=torch.float64, requires_grad=True)
    i = torch.arange(Nq)[:, None] + q_start
    mask = torch.arange(N)[None, :] <= i
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(0, 2, 1, 3), kt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3),
        vt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3), attn_mask=mask)
    g = torch.tensor(x["dout"].reshape(B, Nq, Hq, d), dtype=torch.float64).permute(0, 2, 1, 3)
    (o * g).sum().backward()
    np.testing.assert_allclose(dq.reshape(B, Nq, Hq, d), qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-11)


def test_attn_bwd_closed_form_sums():
    """Per row and head the weights sum to 1 and the logit gradients of eq. (11) sum to
    g.o - g.o = 0, so summed over all keys dV[b, :, r] equals the sum of dout over the group's
    heads and rows, and dK[b, :, r] sums to zero (any selection)."""
    rng = np.random.default_rng(23)
    B, Nq, Hq, Hkv, d = 2, 120, 4, 2, 8
    sh, x = _bwd_case(rng, B=B, N=180, Nq=Nq, q_start=60, Hq=Hq, Hkv=Hkv, d=d, topk=2)
    dq, dk, dv = oracle.attn_bwd(sh, x["q"], x["k"], x["v"], x["ids"], x["dout"])
    G = Hq // Hkv
    dout = x["dout"].astype(np.float64).reshape(B, Nq, Hkv, G, d)
    np.testing.assert_allclose(dv.sum(axis=1), dout.sum(axis=(1, 3)), atol=1e-10)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-10)


def test_idx_bwd_is_finite_difference_of_kl():
    """"KL alignment" §3 / indexer note §2.1: with the selection fixed, the gradient of
    sum(kl_rows) in q_idx and k_idx is the chain of dlogits = P_idx - P through
    S_idx = q_idx.k_idx/sqrt(d_idx) (one shared k_idx head); central differences of the
    oracle's own KL on fp32 inputs."""
    rng = np.random.default_rng(24)
    sh, x = _bwd_case(rng, B=1, N=160, Nq=80, q_start=80, Hq=4, Hkv=2, d=8, di=4, topk=2)
    base = oracle.kl(sh, x["q"], x["k"], x["q_idx"], x["k_idx"], x["ids"])
    dqi, dki = oracle.idx_bwd(sh, x["q_idx"], x["k_idx"], x["ids"], base["dlogits"], coef=1.0)

    def total(qi, ki):
        return float(oracle.kl(sh, x["q"], x["k"], qi, ki, x["ids"],
                               want_dlogits=False)["kl_rows"].sum())

    for name, grad in (("q_idx", dqi), ("k_idx", dki)):
        a = x[name]
        for _ in range(10):
            idx = tuple(int(rng.integers(0, s)) for s in a.shape)
            p, m = a.copy(), a.copy()
            p[idx] = np.float32(a[idx] + np.float32(2e-3))
            m[idx] = np.float32(a[idx] - np.float32(2e-3))
            args = {"qi": x["q_idx"], "ki": x["k_idx"]}
            key = "qi" if name == "q_idx" else "ki"
            f = (total(**{**args, key: p}) - total(**{**args, key: m})) / (float(p[idx]) - float(m[idx]))
            assert abs(f - grad[idx]) < 2e-5 * max(1.0, abs(f)), (name, idx, f, grad[idx])


# ----------------------------------------------------------------------- FP8 index scoring


def _e4m3_grid():
    """Every finite non-negative E4M3 value (OCP: bias 7, 3 mantissa bits, max 448)."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    vals += [(1 + m / 8) * 2.0 ** (E - 7) for E in range(1, 16) for m in range(8)
             if not (E == 15 and m == 7)]
    return np.array(vals)


def test_e4m3_encode_matches_torch_float8_e4m3fn():
    """The oracle's E4M3 rounding (nearest value, ties to the even code) equals torch's
    float8_e4m3fn conversion bit for bit: random fp32 values over the whole range
    (subnormals included, both signs), every exact midpoint between neighbouring codes,
    and the codes themselves."""
    rng = np.random.default_rng(31)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 4000))
    vals = (mag * rng.choice([-1.0, 1.0], 4000)).astype(np.float32)
    grid = _e4m3_grid()
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    allv = np.concatenate([vals, mids, -mids, grid.astype(np.float32), np.float32([0.0, -0.0])])
    ref = torch.from_numpy(allv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(allv.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    # decode is the inverse on every code, and the spec's landmarks
    codes = np.arange(0x7F, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_decode(codes), grid)
    assert oracle.e4m3_encode([448.0, 2.0 ** -6, 2.0 ** -9, 1.0]).tolist() == [0x7E, 0x08, 0x01,
                                                                              0x38]


def test_fp8_scale_exponent_is_the_smallest_fit():
    """e = the smallest integer with amax <= 448 * 2^e, checked by brute force on either side
    of powers of two and on random magnitudes."""
    rng = np.random.default_rng(32)
    tests = list(np.exp2(rng.uniform(-30, 30, 500)))
    tests += [448.0 * 2.0 ** k for k in range(-20, 20)]
    tests += [np.nextafter(448.0 * 2.0 ** k, np.inf) for k in range(-20, 20)]
    for a in tests:
        e = oracle.fp8_scale_exp(a)
        assert a <= 448.0 * 2.0 ** e and not (a <= 448.0 * 2.0 ** (e - 1)), (a, e)
    assert oracle.fp8_scale_exp(0.0) == 0


def test_select_fp8_equals_exact_selection_on_representable_inputs():
    """When every Q_idx row and K_idx block is an E4M3 value times the power of two that the
    scale rule picks (here: each row and block holds one +-448 * 2^e entry), quantization is
    exact and the FP8 path must reproduce the exact selection, scores and margin. The K_idx
    blocks get different exponents, so a per-tensor or per-token scale would not be exact."""
    rng = np.random.default_rng(33)
    N, Nq, q_start, Bk, Hkv, di, k = 300, 120, 180, 32, 2, 8, 3
    nb = (N + Bk - 1) // Bk
    grid = _e4m3_grid()

    def draw(*shape):
        v = rng.choice(grid[40:], size=shape) * rng.choice([-1.0, 1.0], size=shape)
        return v

    q = draw(Nq, Hkv, di)
    q[..., 0] = 448.0
    q *= np.exp2(rng.integers(-6, 3, size=(Nq, Hkv, 1)))
    kk = draw(1, N, di)
    for b in range(nb):
        kk[0, b * Bk, 0] = -448.0
        kk[0, b * Bk:(b + 1) * Bk] *= 2.0 ** (-(b % 5))
    q, kk = q.astype(np.float32), kk.astype(np.float32)
    sh = shape(seqlen_kv=N, seqlen_q=Nq, q_start=q_start, num_kv_heads=Hkv, idx_dim=di,
               block_size=Bk, topk=k)
    qz = oracle.quantize_fp8(sh, q, kk)
    assert qz["k_exp"][0].tolist() == [-(b % 5) for b in range(nb)]
    np.testing.assert_array_equal(oracle.e4m3_decode(qz["k8"]) * np.exp2(
        np.repeat(qz["k_exp"], Bk, axis=1)[:, :N, None]), kk)
    exact = oracle.select(sh, q, kk, want_scores=True, want_margin=True)
    f8 = oracle.select_fp8(sh, qz["q8"], qz["q_exp"], qz["k8"], qz["k_exp"], want_scores=True,
                           want_margin=True)
    np.testing.assert_array_equal(f8["ids"], exact["ids"])
    np.testing.assert_array_equal(f8["block_scores"], exact["block_scores"])
    np.testing.assert_array_equal(f8["margin"], exact["margin"])
