"""GPU parity of the FP8 index branch (msa_index_quantize_fp8, msa_select_fp8) and the
churn of the FP8 selection against the bf16 one.

"MSA Indexer 与 DSA Lightning Indexer 的差别" §3.1: the indexer may run in FP8;
"4.1.1 · 监督与联合训练" after eq. (9): a small cutoff margin Delta lets FP8
quantization flip candidates.

Parity: the quantized bytes and exponents equal the oracle's (bit-exact, every
element); block scores are within 5e-4 of the oracle's exact fp64 sums of the
same E4M3 products (the FP8 matrix cores' sums are not exact fp32: a probe
found errors up to 2^-9 on sums near 100, about 2e-5 relative); ids bit-exact
except rows whose oracle margin is below 1e-3, which must still be valid.

Churn (FP8 vs bf16 on the GPU, every row): with eps = the row's largest block
score difference between the two paths, a row can only change its selection
if its bf16 cutoff margin is <= 2 eps. The share of changed rows per margin
bin is printed (the report of the selector supervision page's eq. 9).
"""
import json

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu

SCORE_TOL = 5e-4
NEAR = 1e-3


def _cfg(name, **kw):
    return si.CONFIGS["main_n8192"].replace(name=name, seed=19).replace(**kw)


CASES = [
    si.CONFIGS["tiny_f32_n1024"],
    _cfg("bf16_g16_ragged", seqlen_kv=1000, seqlen_q=1000),
    _cfg("bf16_chunk_d32", batch=2, seqlen_kv=1500, seqlen_q=300, q_start=1200, num_q_heads=16,
         num_kv_heads=2, head_dim=64, idx_dim=32, topk=5),
    _cfg("bf16_hkv1_k20", seqlen_kv=3000, seqlen_q=3000, num_q_heads=4, num_kv_heads=1, topk=20),
    _cfg("bf16_decode_b3", batch=3, seqlen_kv=3000, seqlen_q=1, q_start=2999, topk=6),
    _cfg("bf16_decode_hkv8_d32", batch=2, seqlen_kv=2000, seqlen_q=1, q_start=1999,
         num_q_heads=16, num_kv_heads=8, idx_dim=32, topk=4),
    # prefill at Hkv=8: 48 queries per 384-row FP8 index tile, ragged N=1000, two sequences
    _cfg("bf16_hkv8_prefill", batch=2, seqlen_kv=1000, seqlen_q=1000, num_q_heads=16,
         num_kv_heads=8, topk=5),
]


def _gpu_fp8(cfg, x, want=True):
    import learned_kv_block_amd as msa
    qz = msa.msa_index_quantize_fp8(x["q_idx"], x["k_idx"], q_start=cfg.q_start,
                                    num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    sel = msa.msa_select_fp8(qz["q8"], qz["q_exp"], qz["k8"], qz["k_exp"], cfg.topk,
                             q_start=cfg.q_start, want_scores=want, want_margin=want,
                             num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    torch.cuda.synchronize()
    return qz, sel


def _check_quantized(cfg, qz, rows, q_idx, k_idx, rep):
    shp = oracle.shape_of(cfg)
    ref = oracle.quantize_fp8(shp, q_idx, k_idx)
    ridx = torch.from_numpy(rows).to(qz["q8"].device)
    H, DI = cfg.num_kv_heads, cfg.idx_dim
    np.testing.assert_array_equal(qz["q8"].reshape(-1, H, DI)[ridx].cpu().numpy(), ref["q8"])
    np.testing.assert_array_equal(qz["q_exp"].reshape(-1, H)[ridx].cpu().numpy(), ref["q_exp"])
    np.testing.assert_array_equal(qz["k8"].cpu().numpy(), ref["k8"])
    np.testing.assert_array_equal(qz["k_exp"].cpu().numpy(), ref["k_exp"])
    rep["bytes_checked"] = int(ref["q8"].size + ref["k8"].size)
    return ref


def _check_select(cfg, sel, rows, refq, lrows, shp, rep):
    ref = oracle.select_fp8(shp, refq["q8"], refq["q_exp"], refq["k8"], refq["k_exp"], rows=lrows,
                            want_scores=True, want_margin=True)
    H, nb = cfg.num_kv_heads, cfg.num_blocks
    ridx = torch.from_numpy(rows).to(sel["ids"].device)
    gsc = sel["block_scores"].reshape(-1, H, nb)[ridx].cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref["block_scores"])  # the causal part (the rest is not written)
    err = float(np.max(np.abs(gsc[fin] - ref["block_scores"][fin])))
    rep["block_scores_max_abs"] = err
    assert err <= SCORE_TOL, err
    gids = sel["ids"].reshape(-1, H, cfg.topk)[ridx].cpu().numpy()
    parity.check_ids(cfg, gids, ref, rep, near_tie=NEAR)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_fp8_every_row(cfg):
    print(f"[fp8] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg, names=("q_idx", "k_idx"))
    qz, sel = _gpu_fp8(cfg, x)
    rows = np.arange(cfg.batch * cfg.seqlen_q, dtype=np.int64)
    q_idx = si.host_query_rows(cfg, "q_idx", rows)
    k_idx = si.host_tensor(cfg, "k_idx")
    rep = {}
    refq = _check_quantized(cfg, qz, rows, q_idx, k_idx, rep)
    _check_select(cfg, sel, rows, refq, None, oracle.shape_of(cfg), rep)
    print(f"[fp8] {cfg.name}: " + json.dumps(rep), flush=True)


# the skewed 131072 workload, and the largest supported sequence (2048 blocks) at Hkv=8
FP8_FULL = [si.CONFIGS["skewed_n131072"],
            _cfg("fp8_prefill_max", seqlen_kv=262144, seqlen_q=262144, num_q_heads=16,
                 num_kv_heads=8, topk=16)]


@pytest.mark.parametrize("cfg", FP8_FULL, ids=[c.name for c in FP8_FULL])
def test_fp8_full_size_sampled(cfg):
    """Every K_idx byte and exponent, Q_idx bytes and the selection on sampled rows
    against the oracle."""
    print(f"[fp8] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg, names=("q_idx", "k_idx"))
    qz, sel = _gpu_fp8(cfg, x)
    rows = parity.sample_rows(cfg, n_random=24, seed=9)
    q_idx = si.host_query_rows(cfg, "q_idx", rows)
    k_idx = si.host_tensor(cfg, "k_idx")
    rep = {}
    shp = oracle.shape_of(cfg)
    refq = oracle.quantize_fp8(shp, q_idx, k_idx)
    ridx = torch.from_numpy(rows).to(qz["q8"].device)
    H, DI = cfg.num_kv_heads, cfg.idx_dim
    np.testing.assert_array_equal(qz["q8"].reshape(-1, H, DI)[ridx].cpu().numpy(), refq["q8"])
    np.testing.assert_array_equal(qz["q_exp"].reshape(-1, H)[ridx].cpu().numpy(), refq["q_exp"])
    np.testing.assert_array_equal(qz["k8"].cpu().numpy(), refq["k8"])
    np.testing.assert_array_equal(qz["k_exp"].cpu().numpy(), refq["k_exp"])
    _check_select(cfg, sel, rows, refq, rows, shp, rep)
    print(f"[fp8] {cfg.name}: " + json.dumps(rep), flush=True)


@pytest.mark.parametrize("di", [64, 32])
def test_fp8_decode_matches_prefill(di):
    """One query per sequence runs the register-streamed FP8 scan; it issues the tiled
    kernel's instruction on the same bytes, so one decode step at the last position gives
    the last prefill row's FP8 block scores and ids bit for bit."""
    import learned_kv_block_amd as msa
    cfg = _cfg(f"fp8_dec_vs_pre_di{di}", batch=2, seqlen_kv=2100, seqlen_q=2100, idx_dim=di,
               num_kv_heads=4 if di == 64 else 8, num_q_heads=64, topk=6)
    x = parity.gpu_inputs(cfg, names=("q_idx", "k_idx"))
    _, pre = _gpu_fp8(cfg, x)
    dcfg = cfg.replace(seqlen_q=1, q_start=cfg.seqlen_kv - 1)
    xd = {"q_idx": x["q_idx"][:, -1:].contiguous(), "k_idx": x["k_idx"]}
    _, dec = _gpu_fp8(dcfg, xd)
    nbl = (cfg.seqlen_kv - 1) // 128 + 1
    H = cfg.num_kv_heads
    sd = dec["block_scores"].reshape(cfg.batch, H, -1)[..., :nbl]
    sp = pre["block_scores"].reshape(cfg.batch, cfg.seqlen_q, H, -1)[:, -1, :, :nbl]
    assert torch.equal(sd, sp)
    assert torch.equal(dec["ids"][:, 0], pre["ids"][:, -1])
    assert torch.equal(dec["margin"][:, 0], pre["margin"][:, -1])


# 64 x 131072, and two sequences at the largest supported cache (2048 blocks, Hkv=8)
FP8_DECODE_FULL = [si.CONFIGS["decode_b64_n131072"],
                   _cfg("fp8_decode_max", batch=2, seqlen_kv=262144, seqlen_q=1,
                        q_start=262143, num_q_heads=16, num_kv_heads=8, topk=16)]


@pytest.mark.parametrize("cfg", FP8_DECODE_FULL, ids=[c.name for c in FP8_DECODE_FULL])
def test_fp8_decode_full_size(cfg):
    """Decode with the FP8 index: every K_idx byte and exponent, and every sequence's
    selection against the oracle (K_idx generated 8 sequences at a time)."""
    print(f"[fp8] start {cfg.name}", flush=True)
    x = parity.gpu_inputs(cfg, names=("q_idx", "k_idx"))
    qz, sel = _gpu_fp8(cfg, x)
    rep = {"rows_checked": 0}
    H, DI = cfg.num_kv_heads, cfg.idx_dim
    for b0 in range(0, cfg.batch, 8):
        rows = np.arange(b0, min(cfg.batch, b0 + 8), dtype=np.int64)  # row = sequence
        lrows = np.arange(len(rows), dtype=np.int64)
        shp = oracle.shape_of(cfg.replace(batch=len(rows)))
        refq = oracle.quantize_fp8(shp, si.host_query_rows(cfg, "q_idx", rows),
                                   si.host_batch_rows(cfg, "k_idx", rows))
        ridx = torch.from_numpy(rows).to(qz["q8"].device)
        np.testing.assert_array_equal(qz["q8"].reshape(-1, H, DI)[ridx].cpu().numpy(), refq["q8"])
        np.testing.assert_array_equal(qz["q_exp"].reshape(-1, H)[ridx].cpu().numpy(),
                                      refq["q_exp"])
        np.testing.assert_array_equal(qz["k8"][b0:b0 + len(rows)].cpu().numpy(), refq["k8"])
        np.testing.assert_array_equal(qz["k_exp"][b0:b0 + len(rows)].cpu().numpy(),
                                      refq["k_exp"])
        part = {}
        _check_select(cfg, sel, rows, refq, lrows, shp, part)
        rep["rows_checked"] += len(rows) * H
        rep["block_scores_max_abs"] = max(rep.get("block_scores_max_abs", 0.0),
                                          part["block_scores_max_abs"])
        print(f"[fp8] {cfg.name} sequences {b0}..{rows[-1]} ok", flush=True)
    assert rep["rows_checked"] == cfg.batch * H
    print(f"[fp8] {cfg.name}: " + json.dumps(rep), flush=True)


def churn_report(cfg, x):
    """FP8 vs bf16 selection on every row (GPU values): changed-row share overall and per
    bf16 cutoff-margin bin, set overlap, and the eq.-(9) bound check."""
    import learned_kv_block_amd as msa
    s16 = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start, want_scores=True,
                         want_margin=True, num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim)
    _, s8 = _gpu_fp8(cfg, x)
    ids16, ids8 = s16["ids"], s8["ids"]
    changed = (ids16 != ids8).any(dim=-1)
    m16, m8 = s16["block_scores"], s8["block_scores"]
    dev = m16.device
    L = (cfg.q_start + torch.arange(cfg.seqlen_q, device=dev)) // 128
    fin = (torch.arange(cfg.num_blocks, device=dev).view(1, 1, 1, -1) <= L.view(1, -1, 1, 1))
    fin = fin.expand_as(m16)  # the causal part (the rest is not written)
    diff = torch.where(fin, (m8 - m16).abs(), torch.zeros_like(m16))
    eps = diff.amax(dim=-1)
    margin = s16["margin"]
    finite_m = torch.isfinite(margin)
    bad = changed & finite_m & (margin > 2 * eps + 1e-6)
    inter = torch.zeros_like(changed, dtype=torch.float32)
    k = cfg.topk
    for s in range(k):  # |S8 ∩ S16| (ids ascending, distinct, -1 padded)
        inter += ((ids8[..., s:s + 1] == ids16) & (ids16 >= 0)).any(dim=-1).float()
    nsel = (ids16 >= 0).sum(dim=-1).float()
    bins = [0.0, 0.01, 0.03, 0.1, 0.3, float("inf")]
    per_bin = {}
    for lo, hi in zip(bins[:-1], bins[1:]):
        sel_rows = finite_m & (margin >= lo) & (margin < hi)
        n = int(sel_rows.sum())
        per_bin[f"[{lo},{hi})"] = {"rows": n,
                                   "changed": float(changed[sel_rows].float().mean()) if n else 0.0}
    return {"rows": int(changed.numel()), "changed_share": float(changed.float().mean()),
            "overlap_mean": float((inter / nsel.clamp(min=1)).mean()),
            "score_diff_max": float(eps.max()), "score_diff_mean": float(diff[fin].mean()),
            "by_bf16_margin": per_bin, "bound_violations": int(bad.sum())}


@pytest.mark.parametrize("name", ["main_n8192", "skewed_n131072"])
def test_fp8_churn_vs_bf16(name):
    cfg = si.CONFIGS[name]
    print(f"[fp8] churn {name}", flush=True)
    x = parity.gpu_inputs(cfg, names=("q_idx", "k_idx"))
    rep = churn_report(cfg, x)
    print(f"[fp8] churn {name}: " + json.dumps(rep), flush=True)
    assert rep["bound_violations"] == 0
