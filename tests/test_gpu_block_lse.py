"""GPU parity of msa_index_block_lse (through the C ABI) against the fp64 oracle.

The index forward with per-block log-sum-exp ("MSA 中的 KL 对齐与局部知识蒸馏" (KL
alignment note) §6): block_lse[i, r, b] = log of the sum over keys j <= i of block b
of exp(S_idx[i, r, j]). Three checks per workload:
  - block_scores equal msa_select's bit for bit (the same products; max is exact);
  - block_lse against the oracle's block_lse: max-abs <= 1e-5 * max(1, |ref|). The
    GPU logits are fp32 sums of 64 bf16 products (relative error ~1e-6 of |s|) and
    the exponentials and logarithm are the hardware's (about one ulp); dropping one
    key of a block moves its LSE by about 1/128, far above the bar;
  - the two routes to the student's LSE_idx agree on the GPU's own selection: the
    log-sum-exp over the selected blocks of the GPU's block_lse equals the oracle's
    lse_idx, which is computed directly over the support (same bar; seen: <= 1e-6).
Blocks past each row's local block must be -inf in both outputs.
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
    base = si.CONFIGS["main_n8192"].replace(name=name, seed=17)
    return base.replace(**kw)


CASES = [
    si.CONFIGS["tiny_f32_n1024"],
    _cfg("bf16_g16_ragged", seqlen_kv=1000, seqlen_q=1000, num_q_heads=64, num_kv_heads=4,
         topk=4),
    _cfg("bf16_chunk_di32", batch=2, seqlen_kv=1500, seqlen_q=300, q_start=1200,
         num_q_heads=16, num_kv_heads=2, head_dim=64, idx_dim=32, topk=5),
    _cfg("bf16_hkv8", seqlen_kv=700, seqlen_q=700, num_q_heads=16, num_kv_heads=8, topk=3),
    _cfg("bf16_hkv1", seqlen_kv=900, seqlen_q=900, num_q_heads=16, num_kv_heads=1, topk=5),
    _cfg("bf16_decode", batch=3, seqlen_kv=3000, seqlen_q=1, q_start=2999, num_q_heads=64,
         num_kv_heads=4, topk=6),
]


def _lse(x, axis=-1):
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        return np.squeeze(m, axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def _check(cfg, rows, res, sel, rep):
    Hkv, nb = cfg.num_kv_heads, (cfg.seqlen_kv + 127) // 128
    sub, lrows, h = parity.host_inputs_for_rows(cfg, rows)
    shp = oracle.shape_of(sub)
    ref = oracle.select(shp, h["q_idx"], h["k_idx"], rows=lrows, want_lse=True)
    ridx = torch.from_numpy(rows).to(res["block_lse"].device)
    gl = res["block_lse"].reshape(-1, Hkv, nb)[ridx].cpu().numpy().astype(np.float64)
    gs = res["block_scores"].reshape(-1, Hkv, nb)[ridx]
    ss = sel["block_scores"].reshape(-1, Hkv, nb)[ridx]
    t = (rows % cfg.seqlen_q) + cfg.q_start
    causal = np.arange(nb)[None, None, :] <= (t // 128)[:, None, None]
    causal_t = torch.from_numpy(causal).to(gs.device).expand_as(gs)
    assert torch.equal(gs[causal_t], ss[causal_t]), "block scores differ from msa_select"
    assert bool(torch.isneginf(gs[~causal_t]).all()), "scores past the local block"
    assert np.all(np.isneginf(gl[~np.broadcast_to(causal, gl.shape)])), "LSE past the local block"
    rl = ref["block_lse"]
    cm = np.broadcast_to(causal, gl.shape)
    err = float(np.max(np.abs(gl[cm] - rl[cm])))
    bar = 1e-5 * max(1.0, float(np.max(np.abs(rl[cm]))))
    rep["block_lse_max_abs"] = err
    assert err <= bar, f"block_lse max-abs {err:.3g} > {bar:.3g}"
    # R16: logsumexp over the selected blocks of the block LSEs = lse_idx over J
    gids = sel["ids"].reshape(-1, Hkv, cfg.topk)[ridx].cpu().numpy()
    kref = oracle.kl(shp, h["q"], h["k"], h["q_idx"], h["k_idx"], gids, rows=lrows,
                     want_dlogits=False)
    picked = np.where(gids >= 0, np.take_along_axis(gl, np.maximum(gids, 0), axis=2), -np.inf)
    two = _lse(picked)
    err2 = float(np.max(np.abs(two - kref["lse_idx"])))
    bar2 = 1e-5 * max(1.0, float(np.max(np.abs(kref["lse_idx"]))))
    rep["route_lse_idx_max_abs"] = err2
    assert err2 <= bar2, f"two-route LSE_idx max-abs {err2:.3g} > {bar2:.3g}"


def _run(cfg):
    import learned_kv_block_amd as msa
    x = parity.gpu_inputs(cfg, names=("q_idx", "k_idx"))
    res = msa.msa_index_block_lse(x["q_idx"], x["k_idx"], q_start=cfg.q_start,
                                  num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start,
                         want_scores=True, num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    torch.cuda.synchronize()
    return res, sel


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_block_lse_every_row(cfg):
    print(f"[block_lse] start {cfg.name}", flush=True)
    res, sel = _run(cfg)
    rows = np.arange(cfg.batch * cfg.seqlen_q, dtype=np.int64)
    rep = {}
    _check(cfg, rows, res, sel, rep)
    print(f"[block_lse] {cfg.name}: " + json.dumps(rep), flush=True)


def test_block_lse_full_size_sampled():
    """Skewed routing at N = 131072 (hot blocks, boosted query rows), sampled rows."""
    cfg = si.CONFIGS["skewed_n131072"]
    print(f"[block_lse] start {cfg.name}", flush=True)
    res, sel = _run(cfg)
    rows = parity.sample_rows(cfg, n_random=16, seed=5)
    rep = {}
    _check(cfg, rows, res, sel, rep)
    print(f"[block_lse] {cfg.name}: " + json.dumps(rep), flush=True)
    del res, sel
    torch.cuda.empty_cache()
