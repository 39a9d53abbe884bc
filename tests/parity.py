"""Helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (checked element by element):
  fp32 workloads: max-abs 1e-5 on outputs, LSE, KL rows and the KL gradient;
  bf16 workloads: max-abs 1e-2 and relative L2 <= 5e-3 (fp32 accumulation);
  block scores: max-abs 1e-5 (fp32) / 1e-4 (bf16 inputs, fp32 sums of 64 exact
  products against fp64);
  block ids: bit-exact, except rows whose oracle cutoff margin is < 1e-4
  (near ties), which are counted and must still be a valid selection within
  1e-4 of the oracle's cutoff.
Outputs, LSE and KL are compared against the oracle evaluated on the GPU's
ids, so they measure the attention and KL arithmetic alone.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import seeded_inputs as si

NEAR_TIE = 1e-4


def tol(cfg):
    if cfg.dtype == si.F32:
        return dict(max_abs=1e-5, rel_l2=None, score=1e-5)
    return dict(max_abs=1e-2, rel_l2=5e-3, score=1e-4)


def gpu_inputs(cfg, names=("q", "k", "v", "q_idx", "k_idx")):
    return {n: si.device_tensor(cfg, n) for n in names}


def run_gpu(cfg, x, want_kl=False, workspace=None):
    import learned_kv_block_amd as msa
    sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start, want_scores=True,
                         want_margin=True, num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    out, lse = msa.msa_attn_fwd(x["q"], x["k"], x["v"], sel["ids"], q_start=cfg.q_start,
                                idx_dim=cfg.idx_dim)
    res = dict(ids=sel["ids"], block_scores=sel["block_scores"], margin=sel["margin"], out=out,
               lse=lse)
    if want_kl:
        kl = msa.msa_kl_align(x["q"], x["k"], x["q_idx"], x["k_idx"], sel["ids"], lse,
                              q_start=cfg.q_start)
        res.update(kl_rows=kl["kl_rows"], kl_mean=kl["kl_mean"], dlogits=kl["dlogits"])
    torch.cuda.synchronize()
    return res


def sample_rows(cfg, n_random=32, seed=0):
    """Query rows (flat b*Nq + t) spanning first rows, block boundaries, the end and random."""
    Nq, B = cfg.seqlen_q, cfg.batch
    rng = np.random.default_rng(seed)
    picks = set()
    for b in range(min(B, 2)):
        for t in [0, 1, 126, 127, 128, 129, 255, 256, Nq // 2, Nq - 129, Nq - 128, Nq - 2, Nq - 1]:
            if 0 <= t < Nq:
                picks.add(b * Nq + t)
    for r in rng.integers(0, B * Nq, size=n_random):
        picks.add(int(r))
    return np.array(sorted(picks), dtype=np.int64)


def host_inputs_for_rows(cfg, rows):
    """Oracle inputs: q, q_idx for the rows; k, v, k_idx for the batches the rows touch."""
    batches = sorted(set(int(r) // cfg.seqlen_q for r in rows))
    bmap = {b: n for n, b in enumerate(batches)}
    q = si.host_query_rows(cfg, "q", rows)
    q_idx = si.host_query_rows(cfg, "q_idx", rows)
    k = si.host_batch_rows(cfg, "k", batches)
    v = si.host_batch_rows(cfg, "v", batches)
    k_idx = si.host_batch_rows(cfg, "k_idx", batches)
    # re-address rows into the compact batch set
    local_rows = np.array([bmap[int(r) // cfg.seqlen_q] * cfg.seqlen_q + int(r) % cfg.seqlen_q
                           for r in rows], dtype=np.int64)
    sub = cfg.replace(batch=len(batches))
    return sub, local_rows, dict(q=q, q_idx=q_idx, k=k, v=v, k_idx=k_idx)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def check_close(name, got, ref, t, report):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    report[name + "_max_abs"] = err
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= t["max_abs"], f"{name}: max-abs {err:.3g} > {t['max_abs']}"
    if t["rel_l2"] is not None and got.size:
        rl = rel_l2(got, ref)
        report[name + "_rel_l2"] = rl
        assert rl <= t["rel_l2"], f"{name}: rel-L2 {rl:.3g} > {t['rel_l2']}"


def check_ids(cfg, gids, ref, report, near_tie=NEAR_TIE):
    """gids, ref['ids'] [n, Hkv, k]; ref has block_scores and margin (fp64). Rows whose
    oracle margin is below near_tie may differ if the GPU's choice is still valid."""
    n, H, k = gids.shape
    near = 0
    for a in range(n):
        for r in range(H):
            g = gids[a, r]
            o = ref["ids"][a, r]
            if np.array_equal(g, o):
                continue
            mg = ref["margin"][a, r]
            assert mg < near_tie, f"row {a} group {r}: ids {g.tolist()} != oracle {o.tolist()} " \
                                  f"(margin {mg:.3g})"
            near += 1
            # still a valid selection: same local block and size, ascending, distinct,
            # every chosen block within NEAR_TIE of the oracle cutoff
            sc = ref["block_scores"][a, r]
            ov = o[o >= 0]
            gv = g[g >= 0]
            assert len(gv) == len(ov) and gv[-1] == ov[-1]
            assert np.all(np.diff(gv) > 0)
            cutoff = min(sc[b] for b in ov[:-1])
            for b in gv[:-1]:
                assert sc[b] >= cutoff - near_tie, (a, r, b, sc[b], cutoff)
    report["near_tie_rows"] = near
    report["rows_checked"] = n * H
    return near


def check_all(cfg, res, rows=None, want_kl=False, report=None):
    """Compare a GPU run with the oracle on `rows` (None = all rows)."""
    report = {} if report is None else report
    t = tol(cfg)
    if rows is None:
        rows = np.arange(cfg.batch * cfg.seqlen_q, dtype=np.int64)
    sub, lrows, h = host_inputs_for_rows(cfg, rows)
    shp = oracle.shape_of(sub)
    ref = oracle.select(shp, h["q_idx"], h["k_idx"], rows=lrows, want_scores=True,
                        want_margin=True)
    Hkv, nb = cfg.num_kv_heads, cfg.num_blocks
    gids = res["ids"].reshape(-1, Hkv, cfg.topk)[torch.from_numpy(rows).to(res["ids"].device)]
    gids = gids.cpu().numpy()
    check_ids(cfg, gids, ref, report)
    # block scores on the causally visible part
    gsc = res["block_scores"].reshape(-1, Hkv, nb)[torch.from_numpy(rows).to(res["ids"].device)]
    gsc = gsc.cpu().numpy().astype(np.float64)
    mask = np.isfinite(ref["block_scores"])
    err = float(np.max(np.abs(gsc[mask] - ref["block_scores"][mask])))
    report["block_scores_max_abs"] = err
    assert err <= t["score"], f"block scores max-abs {err:.3g}"
    gm = res["margin"].reshape(-1, Hkv)[torch.from_numpy(rows).to(res["ids"].device)].cpu().numpy()
    fin = np.isfinite(ref["margin"])
    assert np.array_equal(np.isfinite(gm), fin)
    # the oracle's non-finite margins are +inf (nothing competes for a slot); so must the GPU's be
    assert np.all(np.isposinf(gm[~fin])), "non-finite GPU margins must be +inf"
    if fin.any():
        merr = float(np.max(np.abs(gm[fin] - ref["margin"][fin])))
        report["margin_max_abs"] = merr
        assert merr <= 2 * t["score"] + 1e-6
    # attention on the GPU's ids
    o_ref, l_ref = oracle.attn(shp, h["q"], h["k"], h["v"], gids, rows=lrows)
    dev = res["out"].device
    ridx = torch.from_numpy(rows).to(dev)
    Hq, D = cfg.num_q_heads, cfg.head_dim
    go = res["out"].reshape(-1, Hq, D)[ridx].float().cpu().numpy()
    gl = res["lse"].reshape(-1, Hq)[ridx].cpu().numpy()
    check_close("out", go, o_ref, t, report)
    check_close("lse", gl, l_ref, t, report)
    if want_kl:
        kref = oracle.kl(shp, h["q"], h["k"], h["q_idx"], h["k_idx"], gids, rows=lrows)
        gk = res["kl_rows"].reshape(-1, Hkv)[ridx].cpu().numpy()
        check_close("kl_rows", gk, kref["kl_rows"], t, report)
        gd = res["dlogits"].reshape(-1, Hkv, cfg.topk, 128)[ridx].cpu().numpy()
        check_close("dlogits", gd, kref["dlogits"], t, report)
    return report
