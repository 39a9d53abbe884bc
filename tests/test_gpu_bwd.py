"""GPU parity of msa_attn_bwd (through the C ABI) against the fp64 oracle.

The oracle evaluates eq. (11) of "2.4 · 训练原生稀疏" with the selection held
fixed, on the GPU's own block ids, from the same input bits and the same
seeded upstream gradient dout. Small workloads are checked on every row and
every key; the full-size training workload on sampled rows for dq and, for
dk and dv (sums over every query that selected a block), by the closed-form
key sums: sum over keys of dv equals the sum of dout over the group's heads and
rows, and dk sums to zero (the eq. (11) logit gradients of a row sum to zero).

Tolerances: fp32 relative L2 <= 1e-5; bf16 the forward's bar, relative L2 <= 5e-3
and max-abs <= 1e-2, with the max-abs bar scaled by the largest reference magnitude
where that exceeds 1 (dk and dv sum over every query that chose a block, so their
entries grow with the bucket size, where an absolute 1e-2 would be finer than one
bf16 step of the value). The bf16 kernel rounds P and dS to bf16 for the matrix
cores and writes bf16 per-slot dq partials (each a relative 2^-9 step);
accumulation is fp32.
"""
import json

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu


def _cfg(name, **kw):
    base = si.CONFIGS["main_n8192"].replace(name=name, seed=13)
    return base.replace(**kw)


CASES = [
    si.CONFIGS["tiny_f32_n1024"],
    _cfg("bf16_g16_ragged", seqlen_kv=1000, seqlen_q=1000, num_q_heads=64, num_kv_heads=4,
         topk=4),
    _cfg("bf16_g8_chunk_d64", batch=2, seqlen_kv=1500, seqlen_q=300, q_start=1200,
         num_q_heads=16, num_kv_heads=2, head_dim=64, idx_dim=32, topk=5),
    _cfg("bf16_g1_k20", seqlen_kv=3000, seqlen_q=3000, num_q_heads=4, num_kv_heads=4, topk=20),
    _cfg("bf16_g4_kall", seqlen_kv=900, seqlen_q=900, num_q_heads=16, num_kv_heads=4, topk=12),
    _cfg("bf16_decode_b3", batch=3, seqlen_kv=3000, seqlen_q=1, q_start=2999, num_q_heads=64,
         num_kv_heads=4, topk=6),
    _cfg("f32_g2_short", seqlen_kv=300, seqlen_q=300, num_q_heads=4, num_kv_heads=2,
         head_dim=64, idx_dim=32, topk=2, dtype=si.F32, scale=1.0),
    # bf16 G=2: d=64 with Hkv=8, and d=128 as a chunked prefill starting inside a block
    _cfg("bf16_g2_d64_hkv8", seqlen_kv=700, seqlen_q=700, num_q_heads=16, num_kv_heads=8,
         head_dim=64, topk=3),
    _cfg("bf16_g2_chunk", seqlen_kv=1300, seqlen_q=500, q_start=800, num_q_heads=8,
         num_kv_heads=4, topk=5),
    # two sequences of at least 4096 queries: the forward attention runs one window per
    # sequence, the backward over both at once (ragged last block)
    _cfg("bf16_b2_windows", batch=2, seqlen_kv=4500, seqlen_q=4500, num_q_heads=16,
         num_kv_heads=4, topk=6),
]


def _tol(cfg):
    if cfg.dtype == si.F32:
        return dict(rel_l2=1e-5, max_rel=1e-4, floor=0.0)
    return dict(rel_l2=5e-3, max_rel=1e-2, floor=1.0)


def _check(name, got, ref, t, rep):
    """rel-L2 <= t.rel_l2 and max-abs <= t.max_rel * max(t.floor, max|ref|)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    big = float(np.max(np.abs(ref))) if ref.size else 0.0
    scale = max(big, t["floor"], 1e-30)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    rl = parity.rel_l2(got, ref)
    rep[name] = dict(rel_l2=rl, max_abs=err, max_ref=big)
    assert rl <= t["rel_l2"], f"{name}: rel-L2 {rl:.3g}"
    assert err <= t["max_rel"] * scale, f"{name}: max-abs {err:.3g} (max |ref| {big:.3g})"


def _run(cfg):
    import learned_kv_block_amd as msa
    x = parity.gpu_inputs(cfg, names=("q", "k", "v", "q_idx", "k_idx", "dout"))
    sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start,
                         num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    out, lse = msa.msa_attn_fwd(x["q"], x["k"], x["v"], sel["ids"], q_start=cfg.q_start,
                                idx_dim=cfg.idx_dim)
    dq, dk, dv = msa.msa_attn_bwd(x["q"], x["k"], x["v"], sel["ids"], out, lse, x["dout"],
                                  q_start=cfg.q_start, idx_dim=cfg.idx_dim)
    torch.cuda.synchronize()
    return x, sel["ids"], dq, dk, dv


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_bwd_every_row(cfg):
    print(f"[bwd] start {cfg.name}", flush=True)
    _, ids, dq, dk, dv = _run(cfg)
    n = cfg.batch * cfg.seqlen_q
    rows = np.arange(n, dtype=np.int64)
    shp = oracle.shape_of(cfg)
    q = si.host_query_rows(cfg, "q", rows)
    dout = si.host_query_rows(cfg, "dout", rows)
    k = si.host_tensor(cfg, "k")
    v = si.host_tensor(cfg, "v")
    gids = ids.reshape(n, cfg.num_kv_heads, cfg.topk).cpu().numpy()
    rq, rk, rv = oracle.attn_bwd(shp, q, k, v, gids, dout)
    t = _tol(cfg)
    rep = {}
    _check("dq", dq.float().cpu().numpy().reshape(rq.shape), rq, t, rep)
    _check("dk", dk.float().cpu().numpy(), rk, t, rep)
    _check("dv", dv.float().cpu().numpy(), rv, t, rep)
    print(f"[bwd] {cfg.name}: " + json.dumps(rep), flush=True)


def test_bwd_full_size_sampled():
    """Training workload (2 x 32768 tokens, G=16): dq on sampled rows against the oracle,
    dk and dv by the closed-form key sums."""
    cfg = si.CONFIGS["train_b2_n32768"]
    print(f"[bwd] start {cfg.name}", flush=True)
    x, ids, dq, dk, dv = _run(cfg)
    rows = parity.sample_rows(cfg, n_random=24, seed=3)
    sub, lrows, h = parity.host_inputs_for_rows(cfg, rows)
    dout = si.host_query_rows(cfg, "dout", rows)
    ridx = torch.from_numpy(rows).to(ids.device)
    gids = ids.reshape(-1, cfg.num_kv_heads, cfg.topk)[ridx].cpu().numpy()
    rq, _, _ = oracle.attn_bwd(oracle.shape_of(sub), h["q"], h["k"], h["v"], gids, dout,
                               rows=lrows, want_kv=False)
    t = _tol(cfg)
    rep = {}
    gq = dq.reshape(-1, cfg.num_q_heads, cfg.head_dim)[ridx].float().cpu().numpy()
    _check("dq_sampled", gq, rq, t, rep)
    # closed-form key sums (every query row of the call contributes)
    B, Nq, Hq, D = x["dout"].shape
    Hkv = cfg.num_kv_heads
    G = Hq // Hkv
    want_v = x["dout"].float().reshape(B, Nq, Hkv, G, D).sum(dim=(1, 3))
    got_v = dv.float().sum(dim=1)
    ev = float((got_v - want_v).norm() / want_v.norm())
    got_k = dk.float().sum(dim=1)
    ek = float(got_k.norm() / dk.float().abs().sum(dim=1).norm())
    rep.update(dv_key_sum_rel=ev, dk_key_sum_rel=ek)
    print(f"[bwd] {cfg.name}: " + json.dumps(rep), flush=True)
    assert ev <= 1e-2, ev
    assert ek <= 1e-3, ek


def test_bwd_bitwise_repeatable():
    """Training workload (2 x 32768 tokens): two calls of msa_attn_bwd and of msa_idx_bwd on
    the same inputs give the same bits. Every sum has a fixed order: entries in row order
    inside each bucket, dk / dv / dk_idx slabs of a bucket added in item order (its hot
    buckets span many workgroups), dq and dq_idx partials in slot order."""
    import learned_kv_block_amd as msa
    cfg = si.CONFIGS["train_b2_n32768"]
    print(f"[bwd] start repeatability {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg, names=("q", "k", "v", "q_idx", "k_idx", "dout"))
    sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, num_q_heads=cfg.num_q_heads,
                         head_dim=cfg.head_dim)
    out, lse = msa.msa_attn_fwd(x["q"], x["k"], x["v"], sel["ids"], idx_dim=cfg.idx_dim)
    first = msa.msa_attn_bwd(x["q"], x["k"], x["v"], sel["ids"], out, lse, x["dout"],
                             idx_dim=cfg.idx_dim)
    second = msa.msa_attn_bwd(x["q"], x["k"], x["v"], sel["ids"], out, lse, x["dout"],
                              idx_dim=cfg.idx_dim)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), first, second):
        assert torch.equal(a, b), name
    del first, second
    kl = msa.msa_kl_align(x["q"], x["k"], x["q_idx"], x["k_idx"], sel["ids"], lse)
    ia = msa.msa_idx_bwd(x["q_idx"], x["k_idx"], sel["ids"], kl["dlogits"], 1.0,
                         num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    ib = msa.msa_idx_bwd(x["q_idx"], x["k_idx"], sel["ids"], kl["dlogits"], 1.0,
                         num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    torch.cuda.synchronize()
    assert torch.equal(ia[0], ib[0]), "dq_idx"
    assert torch.equal(ia[1], ib[1]), "dk_idx"
    print(f"[bwd] repeatability {cfg.name}: ok", flush=True)


def test_bwd_bucket_sort_two_passes():
    """140000 query rows: the row-order sort of each bucket takes two passes of its
    131072-row bitmap. Small heads (Hq=2, Hkv=1, d=64, k=2) keep the oracle cheap: dq, dk,
    dv on every row and key, and two calls give the same bits."""
    import learned_kv_block_amd as msa
    cfg = _cfg("bf16_sort_2pass", seqlen_kv=140000, seqlen_q=140000, num_q_heads=2,
               num_kv_heads=1, head_dim=64, idx_dim=32, topk=2)
    print(f"[bwd] start {cfg.name}", flush=True)
    x, ids, dq, dk, dv = _run(cfg)
    out, lse = msa.msa_attn_fwd(x["q"], x["k"], x["v"], ids, idx_dim=cfg.idx_dim)
    again = msa.msa_attn_bwd(x["q"], x["k"], x["v"], ids, out, lse, x["dout"],
                             idx_dim=cfg.idx_dim)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), again):
        assert torch.equal(a, b), name
    n = cfg.batch * cfg.seqlen_q
    rows = np.arange(n, dtype=np.int64)
    q = si.host_query_rows(cfg, "q", rows)
    dout = si.host_query_rows(cfg, "dout", rows)
    gids = ids.reshape(n, cfg.num_kv_heads, cfg.topk).cpu().numpy()
    rq, rk, rv = oracle.attn_bwd(oracle.shape_of(cfg), q, si.host_tensor(cfg, "k"),
                                 si.host_tensor(cfg, "v"), gids, dout)
    t = _tol(cfg)
    rep = {}
    _check("dq", dq.float().cpu().numpy().reshape(rq.shape), rq, t, rep)
    _check("dk", dk.float().cpu().numpy(), rk, t, rep)
    _check("dv", dv.float().cpu().numpy(), rv, t, rep)
    print(f"[bwd] {cfg.name}: " + json.dumps(rep), flush=True)


IDX_CASES = [
    si.CONFIGS["tiny_f32_n1024"],
    _cfg("bf16_g16_idx", seqlen_kv=1000, seqlen_q=1000, num_q_heads=64, num_kv_heads=4, topk=4),
    _cfg("bf16_g8_chunk_d32", batch=2, seqlen_kv=1500, seqlen_q=300, q_start=1200,
         num_q_heads=16, num_kv_heads=2, head_dim=64, idx_dim=32, topk=5),
    _cfg("bf16_decode_idx", batch=3, seqlen_kv=3000, seqlen_q=1, q_start=2999, num_q_heads=64,
         num_kv_heads=4, topk=6),
    # one group (Hkv = 1): every index row shares the one k_idx block accumulator
    _cfg("bf16_hkv1_idx", seqlen_kv=900, seqlen_q=900, num_q_heads=16, num_kv_heads=1, topk=5),
]


@pytest.mark.parametrize("cfg", IDX_CASES, ids=[c.name for c in IDX_CASES])
def test_idx_bwd_every_row(cfg):
    """msa_idx_bwd on the GPU's own ids and dlogits (from msa_kl_align) against the oracle's
    chain of the same dlogits; coef 0.37 checks the scaling."""
    import learned_kv_block_amd as msa
    print(f"[idx_bwd] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg)
    sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start,
                         num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    out, lse = msa.msa_attn_fwd(x["q"], x["k"], x["v"], sel["ids"], q_start=cfg.q_start,
                                idx_dim=cfg.idx_dim)
    kl = msa.msa_kl_align(x["q"], x["k"], x["q_idx"], x["k_idx"], sel["ids"], lse,
                          q_start=cfg.q_start)
    coef = 0.37
    dqi, dki = msa.msa_idx_bwd(x["q_idx"], x["k_idx"], sel["ids"], kl["dlogits"], coef,
                               q_start=cfg.q_start, num_q_heads=cfg.num_q_heads,
                               head_dim=cfg.head_dim)
    torch.cuda.synchronize()
    n = cfg.batch * cfg.seqlen_q
    rows = np.arange(n, dtype=np.int64)
    q_idx = si.host_query_rows(cfg, "q_idx", rows)
    k_idx = si.host_tensor(cfg, "k_idx")
    gids = sel["ids"].reshape(n, cfg.num_kv_heads, cfg.topk).cpu().numpy()
    dl = kl["dlogits"].reshape(n, cfg.num_kv_heads, cfg.topk, 128).cpu().numpy().astype(np.float64)
    rq, rk = oracle.idx_bwd(oracle.shape_of(cfg), q_idx, k_idx, gids, dl, coef=coef)
    t = _tol(cfg)
    rep = {}
    _check("dq_idx", dqi.float().cpu().numpy().reshape(rq.shape), rq, t, rep)
    _check("dk_idx", dki.float().cpu().numpy(), rk, t, rep)
    print(f"[idx_bwd] {cfg.name}: " + json.dumps(rep), flush=True)


def test_idx_bwd_full_size_block_sums():
    """Training workload (2 x 32768 tokens): dk_idx by closed-form block sums. The chain is
    linear in the dlogits, so for every (batch, block) the sum of dk_idx over the block's keys
    equals coef/sqrt(d_idx) times the sum, over the (query, group, slot) that selected the
    block, of that slot's dlogits row sum times the query's q_idx row. Every bucket's slab
    enters these sums: at this size a few buckets start exactly where a workgroup's item
    range starts, whose sums must reach the bucket's own slab."""
    import scipy.sparse
    import learned_kv_block_amd as msa
    cfg = si.CONFIGS["train_b2_n32768"]
    print(f"[idx_bwd] start block sums {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg, names=("q", "k", "v", "q_idx", "k_idx"))
    sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, num_q_heads=cfg.num_q_heads,
                         head_dim=cfg.head_dim)
    out, lse = msa.msa_attn_fwd(x["q"], x["k"], x["v"], sel["ids"], idx_dim=cfg.idx_dim)
    kl = msa.msa_kl_align(x["q"], x["k"], x["q_idx"], x["k_idx"], sel["ids"], lse)
    del out, lse
    coef = 0.37
    _, dki = msa.msa_idx_bwd(x["q_idx"], x["k_idx"], sel["ids"], kl["dlogits"], coef,
                             num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    torch.cuda.synchronize()
    B, Nq, Hkv, K, DI = cfg.batch, cfg.seqlen_q, cfg.num_kv_heads, cfg.topk, cfg.idx_dim
    N, nb = cfg.seqlen_kv, cfg.num_blocks
    n = B * Nq
    ids = sel["ids"].reshape(n * Hkv * K).cpu().numpy()
    # dlogits row sums, one batch at a time on the host
    rs = np.concatenate([kl["dlogits"][b].cpu().numpy().astype(np.float64).sum(axis=-1).ravel()
                         for b in range(B)])
    del kl
    q_idx = si.host_query_rows(cfg, "q_idx", np.arange(n, dtype=np.int64))  # bf16 bits
    qrows = si.bf16_bits_to_f32(q_idx).astype(np.float64).reshape(n * Hkv, DI)
    e = np.nonzero(ids >= 0)[0]
    col = e // K                                     # (b*Nq + t)*Hkv + r
    row = (col // (Nq * Hkv)) * nb + ids[e]          # b*nb + block
    A = scipy.sparse.csr_matrix((rs[e], (row, col)), shape=(B * nb, n * Hkv))
    want = (A @ qrows) * (coef / np.sqrt(DI))
    got = np.zeros((B, nb * 128, DI), np.float64)
    got[:, :N] = dki.float().cpu().numpy()
    got = got.reshape(B, nb, 128, DI).sum(axis=2).reshape(B * nb, DI)
    rep = {}
    _check("dk_idx_block_sums", got, want, _tol(cfg), rep)
    print(f"[idx_bwd] {cfg.name}: " + json.dumps(rep), flush=True)


def test_bwd_empty_rows():
    """No query row: dq and dq_idx are empty; dk, dv and dk_idx (allocated uninitialised
    by the binding) come back zero, since the calls overwrite them."""
    import learned_kv_block_amd as msa
    cfg = _cfg("bf16_empty_bwd", seqlen_kv=512, seqlen_q=0, topk=4)
    x = parity.gpu_inputs(cfg, names=("q", "k", "v", "q_idx", "k_idx", "dout"))
    sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, num_q_heads=cfg.num_q_heads,
                         head_dim=cfg.head_dim)
    out, lse = msa.msa_attn_fwd(x["q"], x["k"], x["v"], sel["ids"], idx_dim=cfg.idx_dim)
    dq, dk, dv = msa.msa_attn_bwd(x["q"], x["k"], x["v"], sel["ids"], out, lse, x["dout"],
                                  idx_dim=cfg.idx_dim)
    dl = torch.zeros((cfg.batch, 0, cfg.num_kv_heads, cfg.topk, 128), dtype=torch.float32,
                     device=x["q"].device)
    dqi, dki = msa.msa_idx_bwd(x["q_idx"], x["k_idx"], sel["ids"], dl,
                               num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and dqi.numel() == 0
    assert dk.shape == x["k"].shape and dv.shape == x["v"].shape and dki.shape == x["k_idx"].shape
    assert bool((dk == 0).all()) and bool((dv == 0).all()) and bool((dki == 0).all())
