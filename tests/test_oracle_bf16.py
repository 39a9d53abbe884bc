"""Pins of the oracle's bf16 input path (dtype = 1: inputs are bf16 bit patterns).

Every bf16 parity claim rests on the oracle reading a bf16 bit pattern as the value
it encodes. These tests tie that decode to facts outside the oracle:
  - known bit patterns with values fixed by the bfloat16 format (sign, 8-bit
    exponent with bias 127, 7 stored mantissa bits), read back as block scores;
  - bit patterns produced by the library's own bfloat16 conversion (torch), whose
    decoded values feed the same fp64 library references as the fp32 pins:
    the masked-matmul block scores, k = all blocks against causal
    scaled_dot_product_attention, and the full-context KL.
A wrong shift, a byte swap or an fp16 decode fails the first test; any decode
that is not the identity on bf16 values fails the others.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def shape(**kw):
    base = dict(batch=1, seqlen_kv=256, seqlen_q=256, q_start=0, num_q_heads=4, num_kv_heads=2,
                head_dim=16, idx_dim=8, block_size=32, topk=3, dtype=1)
    base.update(kw)
    return oracle.RefShape(*[base[f] for f, _ in oracle.RefShape._fields_])


def bf16_pair(rng, *shp, scale=1.0):
    """(bit patterns as uint16, the values they encode as float32), both from torch."""
    x = torch.from_numpy((rng.standard_normal(shp) * scale).astype(np.float32))
    b = x.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16).copy()
    vals = b.to(torch.float32).numpy().copy()
    return bits, vals


# bit pattern -> value, from the bfloat16 format definition
KNOWN = [
    (0x3F80, 1.0),
    (0xBF80, -1.0),
    (0x4000, 2.0),
    (0x3F00, 0.5),
    (0x4049, 3.140625),        # 1.1001001b * 2^1
    (0xC2F7, -123.5),          # -1.1110111b * 2^6
    (0x3C00, 2.0 ** -7),       # an fp16 decode would read 1.0
    (0x0001, 2.0 ** -133),     # smallest subnormal
    (0x0080, 2.0 ** -126),     # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0x0000, 0.0),
]


def test_bf16_known_bit_patterns_read_as_their_values():
    """Each 128-token block holds one token whose K_idx is a known bf16 pattern and filler
    tokens at the lowest finite value; with d_idx = 1 and q_idx = 1.0 the block score is that
    token's value ("MSA Indexer vs DSA" §2.1-§2.2: block score = max of the index logits)."""
    Bk = 128
    nb = len(KNOWN)
    N = nb * Bk
    k_idx = np.full((1, N, 1), 0xFF7F, dtype=np.uint16)  # -(largest finite): the filler
    for b, (bits, _) in enumerate(KNOWN):
        k_idx[0, b * Bk + 5, 0] = bits
    q_idx = np.full((1, 1, 1), 0x3F80, dtype=np.uint16)
    sh = shape(seqlen_kv=N, seqlen_q=1, q_start=N - 1, num_q_heads=1, num_kv_heads=1,
               idx_dim=1, block_size=Bk, topk=2)
    got = oracle.select(sh, q_idx, k_idx, want_scores=True)["block_scores"][0, 0]
    for b, (bits, val) in enumerate(KNOWN):
        assert got[b] == val, (hex(bits), got[b], val)


def test_bf16_and_fp32_paths_agree_on_representable_values():
    """The same values given as bf16 bits (dtype 1) and as fp32 (dtype 0) give identical
    ids, scores, margins, outputs, LSE and KL: the two input paths differ only in decoding."""
    rng = np.random.default_rng(21)
    B, N, Hq, Hkv, d, di, Bk, k = 2, 200, 4, 2, 16, 8, 32, 3
    kw = dict(batch=B, seqlen_kv=N, seqlen_q=N, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
              idx_dim=di, block_size=Bk, topk=k)
    s1, s0 = shape(dtype=1, **kw), shape(dtype=0, **kw)
    q = bf16_pair(rng, B * N, Hq, d)
    kk = bf16_pair(rng, B, N, Hkv, d)
    v = bf16_pair(rng, B, N, Hkv, d)
    qi = bf16_pair(rng, B * N, Hkv, di)
    ki = bf16_pair(rng, B, N, di)
    a = oracle.select(s1, qi[0], ki[0], want_scores=True, want_margin=True)
    b = oracle.select(s0, qi[1], ki[1], want_scores=True, want_margin=True)
    for key in ("ids", "block_scores", "margin"):
        np.testing.assert_array_equal(a[key], b[key])
    oa = oracle.attn(s1, q[0], kk[0], v[0], a["ids"])
    ob = oracle.attn(s0, q[1], kk[1], v[1], b["ids"])
    np.testing.assert_array_equal(oa[0], ob[0])
    np.testing.assert_array_equal(oa[1], ob[1])
    ka = oracle.kl(s1, q[0], kk[0], qi[0], ki[0], a["ids"])
    kb = oracle.kl(s0, q[1], kk[1], qi[1], ki[1], b["ids"])
    np.testing.assert_array_equal(ka["kl_rows"], kb["kl_rows"])
    np.testing.assert_array_equal(ka["dlogits"], kb["dlogits"])


@pytest.mark.parametrize("N,Bk,q_start,Nq", [(200, 32, 0, 200), (300, 64, 120, 100)])
def test_bf16_block_scores_match_masked_matmul(N, Bk, q_start, Nq):
    """"MSA Indexer vs DSA" §2.1-§2.2 on bf16 inputs: block score = max over j in the block
    with j <= i of Q_idx K_idx^T / sqrt(d_idx), against a library fp64 matmul of the values
    torch's bfloat16 conversion encodes."""
    rng = np.random.default_rng(22)
    B, H, di, k = 2, 3, 8, 2
    sh = shape(batch=B, seqlen_kv=N, seqlen_q=Nq, q_start=q_start, num_q_heads=H,
               num_kv_heads=H, idx_dim=di, block_size=Bk, topk=k)
    qb, qv = bf16_pair(rng, B, Nq, H, di)
    kb, kv = bf16_pair(rng, B, N, di)
    out = oracle.select(sh, qb.reshape(B * Nq, H, di), kb, want_scores=True)
    nb = (N + Bk - 1) // Bk
    for b in range(B):
        S = torch.from_numpy(qv[b].astype(np.float64)).reshape(Nq * H, di) @ \
            torch.from_numpy(kv[b].astype(np.float64)).T
        S = (S / math.sqrt(di)).reshape(Nq, H, N).numpy()
        for t in range(Nq):
            i = q_start + t
            for blk in range(nb):
                got = out["block_scores"][b * Nq + t, :, blk]
                if blk * Bk > i:
                    assert np.all(got == -np.inf)
                else:
                    ref = S[t, :, blk * Bk:min(blk * Bk + Bk, i + 1)].max(axis=1)
                    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


def test_bf16_k_all_blocks_is_dense_causal_attention():
    """"2.4 · 训练原生稀疏": k covering every block is full causal attention. bf16 bits through
    select -> attn against the library's causal scaled_dot_product_attention in fp64 on the
    decoded values (GQA with G = 2, ragged last block, chunked prefill)."""
    rng = np.random.default_rng(23)
    B, N, Nq, q_start, Bk = 2, 257, 100, 157, 32
    Hq, Hkv, d, di = 4, 2, 16, 8
    nb = (N + Bk - 1) // Bk
    sh = shape(batch=B, seqlen_kv=N, seqlen_q=Nq, q_start=q_start, num_q_heads=Hq,
               num_kv_heads=Hkv, head_dim=d, idx_dim=di, block_size=Bk, topk=nb)
    qb, qv = bf16_pair(rng, B, Nq, Hq, d)
    kb, kv = bf16_pair(rng, B, N, Hkv, d)
    vb, vv = bf16_pair(rng, B, N, Hkv, d)
    qib, _ = bf16_pair(rng, B * Nq, Hkv, di)
    kib, _ = bf16_pair(rng, B, N, di)
    ids = oracle.select(sh, qib, kib)["ids"]
    o, lse = oracle.attn(sh, qb.reshape(B * Nq, Hq, d), kb, vb, ids)
    G = Hq // Hkv
    qt = torch.from_numpy(qv.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(kv.astype(np.float64)).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(vv.astype(np.float64)).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    mask = torch.arange(N)[None, :] <= (torch.arange(Nq)[:, None] + q_start)
    o_ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    s = (qt @ kt.transpose(-1, -2)) / math.sqrt(d)
    lse_ref = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(o.reshape(B, Nq, Hq, d), o_ref.permute(0, 2, 1, 3).numpy(),
                               atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse.reshape(B, Nq, Hq), lse_ref.permute(0, 2, 1).numpy(),
                               atol=1e-12, rtol=1e-12)


def test_bf16_kl_dense_support_matches_full_context_logits():
    """"KL alignment" §2-§3 on bf16 inputs with k covering every block: the row KL and its
    gradient equal kl_row on logits built by library matmuls of the decoded values."""
    rng = np.random.default_rng(24)
    N, Hq, Hkv, d, di, Bk = 100, 4, 2, 16, 8, 32
    nb = (N + Bk - 1) // Bk
    sh = shape(seqlen_kv=N, seqlen_q=N, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
               idx_dim=di, block_size=Bk, topk=nb)
    qb, qv = bf16_pair(rng, N, Hq, d)
    qib, qiv = bf16_pair(rng, N, Hkv, di)
    kb, kv = bf16_pair(rng, 1, N, Hkv, d)
    kib, kiv = bf16_pair(rng, 1, N, di)
    ids = oracle.select(sh, qib, kib)["ids"]
    out = oracle.kl(sh, qb, kb, qib, kib, ids)
    G = Hq // Hkv
    for t in [0, 1, 31, 32, 70, 99]:
        for r in range(Hkv):
            K = torch.from_numpy(kv[0, :t + 1, r].astype(np.float64))
            Qg = torch.from_numpy(qv[t, r * G:(r + 1) * G].astype(np.float64))
            sm = (Qg @ K.T / math.sqrt(d)).numpy()
            si = (torch.from_numpy(kiv[0, :t + 1].astype(np.float64)) @
                  torch.from_numpy(qiv[t, r].astype(np.float64)) / math.sqrt(di)).numpy()
            ref = oracle.kl_row(sm, si)
            assert abs(out["kl_rows"][t, r] - ref["kl"]) < 1e-12
            np.testing.assert_allclose(out["dlogits"][t, r].reshape(-1)[:t + 1], ref["dS"],
                                       atol=1e-14)
