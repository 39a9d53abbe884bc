"""GPU parity of the warm-up stage on the full causal context (through the C ABI).

"MSA 中的 KL 对齐与局部知识蒸馏" §5: before Top-k routing, the main branch attends
to the whole causal history and the KL support is every j <= i; §8: block recall
and score recall against that full-history teacher.

The oracle is the same fp64 code as for the sparse stage, given the support
"every block 0..floor(i/128)" (oracle.dense_shape / dense_ids): LSE from the
attention oracle, KL rows, LSE_idx and the teacher's block masses from the KL
oracle. Small workloads are checked on every row; the 2 x 32768 training
workload on sampled rows, plus properties on every row (masses sum to 1,
KL >= 0, recalls in [0, 1]).

Tolerances (max-abs): LSE and LSE_idx 1e-5 (fp32 inputs) / 1e-4 (bf16 inputs:
the products are exact, sums are fp32 over up to 32768 keys); KL rows 1e-5 /
1e-4; block masses 1e-5. Block recall is an integer count over |T| and is
compared exactly with the host's count on the GPU's own masses and ids (the
ranking decision taken on the same fp32 values); score recall within 1e-6.
"""
import json

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from oracle import diagnostics as dg
from tests import parity

pytestmark = pytest.mark.gpu


def _cfg(name, **kw):
    return si.CONFIGS["main_n8192"].replace(name=name, seed=17).replace(**kw)


CASES = [
    si.CONFIGS["tiny_f32_n1024"],
    _cfg("bf16_g16_ragged", seqlen_kv=1000, seqlen_q=1000, num_q_heads=64, num_kv_heads=4),
    _cfg("bf16_g8_chunk_d64", batch=2, seqlen_kv=1500, seqlen_q=300, q_start=1200,
         num_q_heads=16, num_kv_heads=2, head_dim=64, idx_dim=32, topk=5),
    _cfg("bf16_g1", seqlen_kv=700, seqlen_q=700, num_q_heads=4, num_kv_heads=4, topk=3),
    _cfg("bf16_g4_kall", seqlen_kv=900, seqlen_q=900, num_q_heads=16, num_kv_heads=4, topk=12),
    _cfg("bf16_g2_hkv8", seqlen_kv=600, seqlen_q=600, num_q_heads=16, num_kv_heads=8, topk=2),
    _cfg("bf16_decode_b3", batch=3, seqlen_kv=3000, seqlen_q=1, q_start=2999, num_q_heads=64,
         num_kv_heads=4, topk=6),
    # fp32 with G >= 8 takes the per-wave index logits with the lane-half split
    _cfg("f32_g8", seqlen_kv=600, seqlen_q=600, num_q_heads=16, num_kv_heads=2, head_dim=64,
         idx_dim=64, topk=3, dtype=si.F32, scale=1.0),
    _cfg("f32_g16_hkv1_d32", seqlen_kv=520, seqlen_q=400, q_start=120, num_q_heads=16,
         num_kv_heads=1, head_dim=64, idx_dim=32, topk=2, dtype=si.F32, scale=1.0),
    _cfg("bf16_g4_hkv1", seqlen_kv=700, seqlen_q=700, num_q_heads=4, num_kv_heads=1, topk=3),
]


def _tol(cfg):
    if cfg.dtype == si.F32:
        return dict(lse=1e-5, kl=1e-5, mass=1e-5)
    return dict(lse=1e-4, kl=1e-4, mass=1e-5)


def _close(name, got, ref, atol, rep):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), name
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    rep[name + "_max_abs"] = err
    assert err <= atol, f"{name}: max-abs {err:.3g} > {atol}"


def _run(cfg, x):
    import learned_kv_block_amd as msa
    lse = msa.msa_dense_lse(x["q"], x["k"], q_start=cfg.q_start, idx_dim=cfg.idx_dim)
    kl = msa.msa_kl_dense(x["q"], x["k"], x["q_idx"], x["k_idx"], lse, q_start=cfg.q_start)
    sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start,
                         num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    rec = msa.msa_block_recall(kl["block_mass"], sel["ids"], q_start=cfg.q_start,
                               seqlen_kv=cfg.seqlen_kv)
    torch.cuda.synchronize()
    return lse, kl, sel["ids"], rec


def _check_recall(cfg, rows, mass, ids, brec, srec, rep):
    """mass [n, Hkv, nb], ids [n, Hkv, k], brec / srec [n, Hkv]: GPU values of the flat query
    rows `rows`."""
    n, H, _ = mass.shape
    worst = 0.0
    for a in range(n):
        i = cfg.q_start + int(rows[a]) % cfg.seqlen_q
        L = i // 128
        m = mass[a].astype(np.float64)
        for r in range(H):
            sel = [int(b) for b in ids[a, r] if 0 <= b <= L]
            want_b = dg.set_recall(sel, m[r, :L + 1], min(cfg.topk, L + 1))
            assert abs(float(brec[a, r]) - want_b) <= 1e-7, (a, r, brec[a, r], want_b)
            want_s = dg.coverage(sel, m[r])
            worst = max(worst, abs(float(srec[a, r]) - want_s))
    rep["score_recall_max_abs"] = worst
    assert worst <= 1e-6


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_dense_every_row(cfg):
    print(f"[dense] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg)
    lse, kl, ids, rec = _run(cfg, x)
    n = cfg.batch * cfg.seqlen_q
    rows = np.arange(n, dtype=np.int64)
    shp = oracle.dense_shape(oracle.shape_of(cfg))
    dids = oracle.dense_ids(shp)
    q = si.host_query_rows(cfg, "q", rows)
    q_idx = si.host_query_rows(cfg, "q_idx", rows)
    k, v, k_idx = (si.host_tensor(cfg, nm) for nm in ("k", "v", "k_idx"))
    _, l_ref = oracle.attn(shp, q, k, v, dids)
    kref = oracle.kl(shp, q, k, q_idx, k_idx, dids, want_dlogits=False, want_mass=True)
    t = _tol(cfg)
    rep = {}
    H = cfg.num_kv_heads
    _close("lse_main", lse.reshape(n, -1).cpu().numpy(), l_ref, t["lse"], rep)
    _close("lse_idx", kl["lse_idx"].reshape(n, H).cpu().numpy(), kref["lse_idx"], t["lse"], rep)
    _close("kl_rows", kl["kl_rows"].reshape(n, H).cpu().numpy(), kref["kl_rows"], t["kl"], rep)
    _close("kl_mean", kl["kl_mean"].cpu().numpy()[0], kref["kl_mean"], t["kl"], rep)
    mass = kl["block_mass"].reshape(n, H, -1).cpu().numpy()
    _close("block_mass", mass, kref["block_mass"], t["mass"], rep)
    gids = ids.reshape(n, H, cfg.topk).cpu().numpy()
    brec = rec["block_recall"].reshape(n, H).cpu().numpy()
    srec = rec["score_recall"].reshape(n, H).cpu().numpy()
    _check_recall(cfg, rows, mass, gids, brec, srec, rep)
    means = rec["means"].cpu().numpy()
    assert abs(means[0] - brec.astype(np.float64).mean()) <= 1e-6
    assert abs(means[1] - srec.astype(np.float64).mean()) <= 1e-6
    rep.update(block_recall_mean=float(means[0]), score_recall_mean=float(means[1]))
    print(f"[dense] {cfg.name}: " + json.dumps(rep), flush=True)


def test_dense_full_size_sampled():
    """Training workload (2 x 32768 tokens, G=16): sampled rows against the oracle; every row
    by the properties that hold at any size."""
    cfg = si.CONFIGS["train_b2_n32768"]
    print(f"[dense] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg)
    lse, kl, ids, rec = _run(cfg, x)
    H = cfg.num_kv_heads
    mass_all = kl["block_mass"]
    rep = {}
    # every row: masses sum to 1, KL >= 0, recalls in range
    msum = mass_all.sum(dim=-1)
    rep["mass_sum_max_dev"] = float((msum - 1.0).abs().max())
    assert rep["mass_sum_max_dev"] <= 1e-3
    rep["kl_min"] = float(kl["kl_rows"].min())
    assert rep["kl_min"] >= -1e-4
    br, sr = rec["block_recall"], rec["score_recall"]
    assert float(br.min()) >= 0.0 and float(br.max()) <= 1.0
    assert float(sr.min()) >= 0.0 and float(sr.max()) <= 1.0 + 1e-3
    # sampled rows against the oracle
    rows = parity.sample_rows(cfg, n_random=12, seed=5)
    sub, lrows, h = parity.host_inputs_for_rows(cfg, rows)
    shp = oracle.dense_shape(oracle.shape_of(sub))
    dids = oracle.dense_ids(shp, rows=lrows)
    _, l_ref = oracle.attn(shp, h["q"], h["k"], h["v"], dids, rows=lrows)
    kref = oracle.kl(shp, h["q"], h["k"], h["q_idx"], h["k_idx"], dids, rows=lrows,
                     want_dlogits=False, want_mass=True)
    ridx = torch.from_numpy(rows).to(lse.device)
    t = _tol(cfg)
    _close("lse_main", lse.reshape(-1, cfg.num_q_heads)[ridx].cpu().numpy(), l_ref, t["lse"], rep)
    _close("lse_idx", kl["lse_idx"].reshape(-1, H)[ridx].cpu().numpy(), kref["lse_idx"],
           t["lse"], rep)
    _close("kl_rows", kl["kl_rows"].reshape(-1, H)[ridx].cpu().numpy(), kref["kl_rows"], t["kl"],
           rep)
    mass = mass_all.reshape(-1, H, cfg.num_blocks)[ridx].cpu().numpy()
    _close("block_mass", mass, kref["block_mass"], t["mass"], rep)
    gids = ids.reshape(-1, H, cfg.topk)[ridx].cpu().numpy()
    brec = br.reshape(-1, H)[ridx].cpu().numpy()
    srec = sr.reshape(-1, H)[ridx].cpu().numpy()
    _check_recall(cfg, rows, mass, gids, brec, srec, rep)
    rep.update(block_recall_mean=float(rec["means"][0]), score_recall_mean=float(rec["means"][1]),
               kl_mean=float(kl["kl_mean"][0]))
    print(f"[dense] {cfg.name}: " + json.dumps(rep), flush=True)


GRAD_CASES = [
    si.CONFIGS["tiny_f32_n1024"],
    _cfg("bf16_g16_ragged", seqlen_kv=1000, seqlen_q=1000, num_q_heads=64, num_kv_heads=4),
    _cfg("bf16_g8_chunk_d64", batch=2, seqlen_kv=1500, seqlen_q=300, q_start=1200,
         num_q_heads=16, num_kv_heads=2, head_dim=64, idx_dim=32, topk=5),
    _cfg("bf16_g2_hkv8", seqlen_kv=600, seqlen_q=600, num_q_heads=16, num_kv_heads=8, topk=2),
    _cfg("bf16_decode_b3", batch=3, seqlen_kv=3000, seqlen_q=1, q_start=2999, num_q_heads=64,
         num_kv_heads=4, topk=6),
    _cfg("f32_g8", seqlen_kv=600, seqlen_q=600, num_q_heads=16, num_kv_heads=2, head_dim=64,
         idx_dim=64, topk=3, dtype=si.F32, scale=1.0),
    _cfg("bf16_g4_hkv1", seqlen_kv=700, seqlen_q=700, num_q_heads=4, num_kv_heads=1, topk=3),
]
COEF = 0.37


def _grad_close(name, got, ref, rep):
    """bf16 chain (dS and operands rounded to bf16, fp32 sums): the forward's bf16 bar,
    rel-L2 <= 5e-3 and max-abs <= 1e-2, the latter scaled by the largest reference
    magnitude where it exceeds 1 (dk_idx sums over every query row that sees a key)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(got)), name
    rl = parity.rel_l2(got, ref)
    big = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    rep[name] = dict(rel_l2=rl, max_abs=err, max_ref=big)
    assert rl <= 5e-3 and err <= 1e-2 * max(1.0, big), (name, rl, err, big)


@pytest.mark.parametrize("cfg", GRAD_CASES, ids=[c.name for c in GRAD_CASES])
def test_dense_grad_every_row(cfg):
    """msa_kl_dense_bwd: dq_idx, dk_idx against the oracle's chain of its own full-context
    dlogits ("KL alignment" §3, §5); KL rows bit-identical to msa_kl_dense."""
    import learned_kv_block_amd as msa
    print(f"[dense-grad] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg)
    lse = msa.msa_dense_lse(x["q"], x["k"], q_start=cfg.q_start, idx_dim=cfg.idx_dim)
    fwd = msa.msa_kl_dense(x["q"], x["k"], x["q_idx"], x["k_idx"], lse, q_start=cfg.q_start)
    g = msa.msa_kl_dense_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], lse, COEF,
                             q_start=cfg.q_start, want_mass=True)
    torch.cuda.synchronize()
    assert torch.equal(g["kl_rows"], fwd["kl_rows"])
    assert torch.equal(g["block_mass"], fwd["block_mass"])
    n = cfg.batch * cfg.seqlen_q
    rows = np.arange(n, dtype=np.int64)
    shp = oracle.dense_shape(oracle.shape_of(cfg))
    dids = oracle.dense_ids(shp)
    q = si.host_query_rows(cfg, "q", rows)
    q_idx = si.host_query_rows(cfg, "q_idx", rows)
    k, k_idx = si.host_tensor(cfg, "k"), si.host_tensor(cfg, "k_idx")
    kref = oracle.kl(shp, q, k, q_idx, k_idx, dids, want_dlogits=True)
    rq, rk = oracle.idx_bwd(shp, q_idx, k_idx, dids, kref["dlogits"], coef=COEF)
    rep = {}
    _grad_close("dq_idx", g["dq_idx"].float().cpu().numpy().reshape(rq.shape), rq, rep)
    _grad_close("dk_idx", g["dk_idx"].float().cpu().numpy(), rk, rep)
    print(f"[dense-grad] {cfg.name}: " + json.dumps(rep), flush=True)


def test_dense_grad_full_size():
    """2 x 32768 (the gradient runs in 8 chunks of 4096 query rows): dq_idx on sampled rows
    against the oracle; dk_idx through identities over every row: <dk_idx, k_idx> equals
    <dq_idx, q_idx> (both are coef * sum dS * z), and the keys' dk_idx sum to 0 (every
    row's dS sums to 0)."""
    import learned_kv_block_amd as msa
    cfg = si.CONFIGS["train_b2_n32768"]
    print(f"[dense-grad] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg)
    lse = msa.msa_dense_lse(x["q"], x["k"], q_start=cfg.q_start, idx_dim=cfg.idx_dim)
    g = msa.msa_kl_dense_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], lse, COEF,
                             q_start=cfg.q_start, want_kl=False)
    torch.cuda.synchronize()
    rep = {}
    dq, dk = g["dq_idx"].double(), g["dk_idx"].double()
    lhs = float((dk * x["k_idx"].double()).sum())
    rhs = float((dq * x["q_idx"].double()).sum())
    rep["dk_k_vs_dq_q_rel"] = abs(lhs - rhs) / max(abs(rhs), 1e-30)
    ksum = dk.sum(dim=1)
    rep["dk_key_sum_rel"] = float(ksum.norm() / dk.abs().sum(dim=1).norm())
    assert rep["dk_k_vs_dq_q_rel"] <= 1e-2, rep
    assert rep["dk_key_sum_rel"] <= 1e-2, rep
    rows = parity.sample_rows(cfg, n_random=6, seed=11)
    sub, lrows, h = parity.host_inputs_for_rows(cfg, rows)
    shp = oracle.dense_shape(oracle.shape_of(sub))
    dids = oracle.dense_ids(shp, rows=lrows)
    kref = oracle.kl(shp, h["q"], h["k"], h["q_idx"], h["k_idx"], dids, rows=lrows,
                     want_dlogits=True)
    rq, _ = oracle.idx_bwd(shp, h["q_idx"], h["k_idx"], dids, kref["dlogits"], coef=COEF,
                           rows=lrows)
    ridx = torch.from_numpy(rows).to(lse.device)
    got = g["dq_idx"].reshape(-1, cfg.num_kv_heads, cfg.idx_dim)[ridx].float().cpu().numpy()
    _grad_close("dq_idx_sampled", got, rq, rep)
    print(f"[dense-grad] {cfg.name}: " + json.dumps(rep), flush=True)
