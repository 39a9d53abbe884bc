"""Benchmark of the MSA layer hot path on one MI355X.

One step = msa_select (index GEMM + causal block max + Top-k) followed by
msa_attn_fwd (bucketing, KV-outer sparse attention, LSE combine) over one
batch of the skewed long-context workload: batch 1, N = 131072, Hq = 64,
Hkv = 4, d = 128, d_idx = 64, 128-token blocks, k = 16, bf16 inputs with
seeded synthetic values (inputs resident in HBM before timing).

Prints one JSON line: query-tokens/s, ms per step, the effective-FLOP MFMA
fraction of the whole layer, every kernel of the step against its own roofline
(MFMA for the index GEMM and the attention, HBM for the Top-k, the bucketing
and the combine), the roofline of the dominant kernel (the KV-outer sparse
attention, timed live with HIP events over the timed steps in the measurement
build; its gathered-Q and partial-output bytes and the counter bytes alongside,
all per launch: a prefill of more than 32768 queries per sequence runs the
attention once per 32768-query window) and the fp64 oracle timed on the host on a
bounded row sample. In `kernels` the work, bytes and times are per step and
`counter_bytes` per launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15  # dense bf16 MFMA, MI355X
PEAK_HBM = 8.0e12   # bytes/s
PEAK_FP8 = 5.0e15   # dense fp8 MFMA, MI355X
CSRC = os.path.join(ROOT, "learned_kv_block_amd", "csrc")
# Per-kernel HBM counter record (FETCH_SIZE / WRITE_SIZE per dispatch, calibrated on a copy),
# written by `bench.py --ingest-counters`; an entry is used only while its kernel's source is
# unchanged.
def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_counters_{workload}.json")


# rocprofv3 kernel-name fragment -> (timer name, source files whose hash ties the counters to
# the code that was measured)
KERNEL_FILES = {
    "index_blockmax_kernel": ("index_blockmax", ["msa_select.hip"]),
    "index_blockmax_fp8_kernel": ("index_fp8", ["msa_fp8.hip"]),
    "topk_kernel": ("topk", ["msa_select.hip"]),
    "bucket_hist_kernel": ("bucket_hist", ["msa_attn.hip"]),
    "bucket_scatter_kernel": ("bucket_scatter", ["msa_attn.hip"]),
    "work_items_kernel": ("work_items", ["msa_attn.hip"]),
    "sparse_attn_pipe_kernel": ("sparse_attn", ["msa_attn.hip"]),
    "combine_local_kernel": ("combine", ["msa_attn.hip"]),
    "decode_index_kernel": ("index_blockmax", ["msa_decode.hip"]),
    "decode_attn_kernel": ("sparse_attn", ["msa_decode.hip"]),
    "kl_main_pipe_kernel": ("kl_main", ["msa_kl.hip"]),
    "attn_bwd_kernel": ("attn_bwd", ["msa_bwd.hip"]),
    "dq_sum_kernel": ("dq_sum", ["msa_bwd.hip"]),
    "idx_bwd_kernel": ("idx_bwd", ["msa_bwd.hip"]),
    "bucket_sort_kernel": ("bucket_sort", ["msa_attn.hip"]),
    "attn_bwd_finalize_kernel": ("bwd_finalize", ["msa_bwd.hip"]),
}


def source_hash(files) -> str:
    # the entry points decide how a step splits into launches (e.g. attention windows),
    # so a counter record also goes stale when msa_api.cpp changes
    h = hashlib.sha256()
    for f in list(files) + ["msa_internal.hpp", "msa_api.cpp"]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def effective_flops(cfg, ids):
    """Index GEMM over the causal triangle + attention on the causally visible tokens of the
    blocks actually selected (from the GPU's ids). Returns (index, attention, attention on
    the local blocks); in bf16 the local blocks run inside the combine kernel, the rest in
    the KV-outer kernel."""
    import torch
    B, Nq, Hkv, G = cfg.batch, cfg.seqlen_q, cfg.num_kv_heads, cfg.group_size
    i = torch.arange(Nq, device=ids.device, dtype=torch.int64) + cfg.q_start
    f_idx = 2.0 * cfg.idx_dim * Hkv * B * float((i + 1).sum().item())
    L = (i // 128).view(1, -1, 1, 1)
    idsl = ids.long()
    full = (idsl >= 0) & (idsl < L)
    loc = idsl == L
    tok_loc = loc.sum(-1) * ((i % 128) + 1).view(1, -1, 1)
    tok = full.sum(-1) * 128 + tok_loc
    f_attn = 4.0 * cfg.head_dim * G * float(tok.sum().item())
    f_loc = 4.0 * cfg.head_dim * G * float(tok_loc.sum().item())
    return f_idx, f_attn, f_loc


def tile_flops(cfg, ids):
    """FLOPs the kernels execute on full 128-token tiles: the index GEMM over every causal
    block 0..floor(i/128), the attention over every selected block."""
    import torch
    B, Nq, Hkv, G = cfg.batch, cfg.seqlen_q, cfg.num_kv_heads, cfg.group_size
    i = torch.arange(Nq, device=ids.device, dtype=torch.int64) + cfg.q_start
    f_idx = 2.0 * cfg.idx_dim * Hkv * B * 128.0 * float((i // 128 + 1).sum().item())
    f_attn = 4.0 * cfg.head_dim * G * 128.0 * float((ids >= 0).sum().item())
    return f_idx, f_attn


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kv_outer_bytes(cfg, ids):
    """Algorithmic HBM bytes of one KV-outer attention launch (bf16), from the GPU's
    selection: per (query, group, non-local selected block) the group's G gathered Q rows
    (G*d*2 B) and the written partial (G*d*2 B of O + G*4 B of LSE); per distinct
    (batch, group, block) bucket its K and V tiles (2*128*d*2 B) once."""
    import torch
    B, Nq, Hkv, G, D = cfg.batch, cfg.seqlen_q, cfg.num_kv_heads, cfg.group_size, cfg.head_dim
    i = torch.arange(Nq, device=ids.device, dtype=torch.int64) + cfg.q_start
    L = (i // 128).view(1, -1, 1, 1)
    idsl = ids.long()
    sel = (idsl >= 0) & (idsl < L)
    n_trip = int(sel.sum().item())
    nb = (cfg.seqlen_kv + 127) // 128
    b = torch.arange(B, device=ids.device).view(-1, 1, 1, 1)
    r = torch.arange(Hkv, device=ids.device).view(1, 1, -1, 1)
    bkt = ((b * Hkv + r) * nb + idsl)[sel]
    n_bkt = int(torch.unique(bkt).numel())
    return n_trip * (2 * G * D * 2 + G * 4) + n_bkt * 2 * 128 * D * 2, n_trip, n_bkt


def host_cpus():
    """(CPUs this process may run on, CPUs the host reports)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return avail, os.cpu_count() or avail


def cpu_baseline(cfg, seconds_target=15.0):
    """fp64 oracle (select + attention) on a seeded sample of query rows, timed on the host."""
    import numpy as np

    import oracle
    import seeded_inputs as si

    threads = oracle.threads()
    avail, reported = host_cpus()
    k = si.host_tensor(cfg, "k")
    v = si.host_tensor(cfg, "v")
    k_idx = si.host_tensor(cfg, "k_idx")
    shp = oracle.shape_of(cfg)
    rng = np.random.default_rng(1234)

    def run(rows):
        q = si.host_query_rows(cfg, "q", rows)
        qi = si.host_query_rows(cfg, "q_idx", rows)
        t0 = time.perf_counter()
        ids = oracle.select(shp, qi, k_idx, rows=rows)["ids"]
        oracle.attn(shp, q, k, v, ids, rows=rows)
        return time.perf_counter() - t0

    # calibrate on a small sample, then size the sample to ~seconds_target
    probe = np.sort(rng.integers(0, cfg.batch * cfg.seqlen_q, size=2 * threads))
    dt = run(probe)
    n = int(max(2 * threads, min(16384, len(probe) * seconds_target / max(dt, 1e-3))))
    rows = np.sort(rng.integers(0, cfg.batch * cfg.seqlen_q, size=n))
    dt = run(rows)
    return {"value": n / dt, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "threads": threads, "host_cpus_available": avail, "host_cpus_reported": reported,
            "cpu_model": cpu_model(),
            "sample": f"{n} seeded uniformly random query rows of the same workload "
                      f"(rows are independent; fp64 select + attention in {dt:.1f} s, "
                      f"OpenMP over rows on {threads} threads)"}


def dense_flops(cfg):
    """Algorithmic work of the warm-up stage over the causal triangle: exponentials and MFMA
    FLOPs of the main-branch LSE pass and of the KL pass (main S again, index logits)."""
    B, Nq, Hq, Hkv = cfg.batch, cfg.seqlen_q, cfg.num_q_heads, cfg.num_kv_heads
    pairs = B * sum(cfg.q_start + t + 1 for t in range(Nq))  # (query, key) pairs, j <= i
    return {"pairs": pairs,
            "lse_flops": 2.0 * cfg.head_dim * Hq * pairs,
            "lse_exps": float(Hq * pairs),
            "kl_flops": 2.0 * (cfg.head_dim * Hq + cfg.idx_dim * Hkv) * pairs,
            "kl_exps": float(Hq * pairs),
            "idx_lse_flops": 2.0 * cfg.idx_dim * Hkv * pairs}


def cpu_baseline_dense(cfg, seconds_target=15.0):
    """fp64 oracle of the warm-up stage (dense LSE + full-context KL with block masses) on a
    seeded sample of query rows, timed on the host."""
    import numpy as np

    import oracle
    import seeded_inputs as si

    threads = oracle.threads()
    k, v, k_idx = (si.host_tensor(cfg, n) for n in ("k", "v", "k_idx"))
    shp = oracle.dense_shape(oracle.shape_of(cfg))
    rng = np.random.default_rng(4321)

    def run(rows):
        q = si.host_query_rows(cfg, "q", rows)
        qi = si.host_query_rows(cfg, "q_idx", rows)
        ids = oracle.dense_ids(shp, rows=rows)
        t0 = time.perf_counter()
        oracle.attn(shp, q, k, v, ids, rows=rows)
        oracle.kl(shp, q, k, qi, k_idx, ids, rows=rows, want_dlogits=False, want_mass=True)
        return time.perf_counter() - t0

    probe = np.sort(rng.integers(0, cfg.batch * cfg.seqlen_q, size=threads))
    dt = run(probe)
    n = int(max(threads, min(4096, len(probe) * seconds_target / max(dt, 1e-3))))
    rows = np.sort(rng.integers(0, cfg.batch * cfg.seqlen_q, size=n))
    dt = run(rows)
    return {"value": n / dt, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} seeded uniformly random query rows of the same workload "
                      f"(fp64 dense attention LSE + full-context KL and block masses in "
                      f"{dt:.1f} s; the oracle also forms the attention output)"}


def dense_main(args):
    """Warm-up stage: main-branch LSE over the full causal context, KL on that context with
    the teacher's block masses, the k-block selection and its block / score recall."""
    import torch

    import learned_kv_block_amd as msa
    import seeded_inputs as si

    cfg = si.CONFIGS[args.workload or "train_b2_n32768"]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    x = {n: si.device_tensor(cfg, n, dev) for n in ("q", "k", "q_idx", "k_idx")}
    sh = msa.shape_for(x["q_idx"], x["k_idx"], cfg.topk, cfg.q_start, cfg.num_q_heads,
                       cfg.head_dim)
    ws_sel = torch.empty(msa.workspace_size(sh, msa.MSA_OP_SELECT), dtype=torch.uint8, device=dev)

    sh_d = msa.make_shape(cfg.batch, cfg.seqlen_kv, cfg.seqlen_q, cfg.q_start, cfg.num_q_heads,
                          cfg.num_kv_heads, cfg.head_dim, cfg.idx_dim, 1, msa.MSA_BF16)
    ws_grad = torch.empty(msa.workspace_size(sh_d, msa.MSA_OP_KL_DENSE_BWD), dtype=torch.uint8,
                          device=dev)
    coef = 1.0 / (cfg.batch * cfg.seqlen_q * cfg.num_kv_heads)  # mean over rows

    def step():
        lse = msa.msa_dense_lse(x["q"], x["k"], q_start=cfg.q_start, idx_dim=cfg.idx_dim)
        kl = msa.msa_kl_dense_bwd(x["q"], x["k"], x["q_idx"], x["k_idx"], lse, coef,
                                  q_start=cfg.q_start, want_mass=True, workspace=ws_grad)
        sel = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start,
                             num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim,
                             workspace=ws_sel)
        rec = msa.msa_block_recall(kl["block_mass"], sel["ids"], q_start=cfg.q_start,
                                   seqlen_kv=cfg.seqlen_kv)
        return kl, rec

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(max(1, args.warmup)):
        kl, rec = step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    with msa.KernelTimer("kl_dense", max_launches=args.steps * 1024) as kt:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            kl, rec = step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / max(1, args.steps)
    kernels = {}
    for name in ("dense_lse", "dense_lse_idx", "kl_dense", "kl_dense_chain", "index_blockmax",
                 "topk", "recall"):
        with msa.KernelTimer(name, max_launches=4096) as t:
            step()
            step()
            torch.cuda.synchronize()
        kernels[name] = round(t.total_ms / 2, 4)  # per step (the KL runs in row chunks)
    print(f"[bench] kernels {kernels}", file=sys.stderr, flush=True)
    w = dense_flops(cfg)
    kl_ms = kt.total_ms / max(1, args.steps)  # per step, summed over the row chunks
    peak_exp = 256 * 4 * 16 / 4 * 2.4e9  # v_exp_f32: a quarter of the 16-lane FP32 rate
    roofline = {"bound": "mfma", "kernel": "kl_dense", "achieved": w["kl_flops"] / (kl_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": w["kl_flops"] / (kl_ms * 1e-3) / PEAK_BF16, "traffic": None,
                "avg_ms": kl_ms, "launches": kt.launches, "launches_per_step": kt.launches // max(1, args.steps),
                "flops_per_launch": w["kl_flops"], "exps_per_launch": w["kl_exps"],
                "note": "per step: the KL pass runs once per chunk of query rows; flops and "
                        "exponentials are per step",
                "exp_frac": w["kl_exps"] / (kl_ms * 1e-3) / peak_exp}
    tokens = cfg.batch * cfg.seqlen_q
    line = {
        "metric": "MSA warm-up KL step (dense LSE + full-context KL and its gradient into "
                  "q_idx/k_idx + block/score recall) query-tokens/s",
        "value": tokens * args.steps / elapsed,
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seqlen_kv,
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "idx_dim": cfg.idx_dim,
                   "block_size": cfg.block_size, "topk": cfg.topk, "parallelism": "none",
                   "dense_warmup": True},
        "work": w,
        "kernel_ms": kernels,
        "kl_mean": float(kl["kl_mean"][0]),
        "block_recall_mean": float(rec["means"][0]),
        "score_recall_mean": float(rec["means"][1]),
        "roofline": roofline,
    }
    del x, ws_sel, ws_grad, kl, rec
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_dense(cfg)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


def step_work(cfg, ids, fp8=False):
    """Algorithmic work of each kernel of one prefill / decode step (bf16, or with the FP8
    index: 1-byte index operands), from the GPU's own selection. Returns
    {timer name: dict(bound, flops | bytes, what)}."""
    import torch

    import seeded_inputs as si
    B, Nq, Hkv, G, D, K = (cfg.batch, cfg.seqlen_q, cfg.num_kv_heads, cfg.group_size,
                           cfg.head_dim, cfg.topk)
    Hq = Hkv * G
    f_idx, f_attn, f_loc = effective_flops(cfg, ids)
    kv_bytes, n_trip, n_bkt = kv_outer_bytes(cfg, ids)
    i = torch.arange(Nq, device=ids.device, dtype=torch.int64) + cfg.q_start
    L = i // 128
    # Top-k reads the block scores of blocks 0..L-1 of rows with more than k visible blocks
    # (the local block is forced) and writes k ids per (query, group)
    m_read = 4 * B * Hkv * int(torch.where(L + 1 > K, L, torch.zeros_like(L)).sum().item())
    rows = B * Nq * Hkv
    n_sel = int((ids >= 0).sum().item())
    rows_q = B * Nq
    work = {
        "index_blockmax": dict(bound="mfma", flops=f_idx,
                               what="2*d_idx*Hkv flops per causally visible (query, key)"),
        "topk": dict(bound="hbm", bytes=m_read + rows * K * 4,
                     what="block scores of blocks 0..L-1 read, k int32 ids written per row"),
        # histogram and scatter read the ids; the scatter writes one entry per selected
        # non-local slot; work items are 16 B each (counted from the entries: 16 queries/item)
        "bucketing": dict(bound="hbm", bytes=2 * rows * K * 4 + n_trip * 4 + (n_trip // 16) * 16,
                          what="ids read twice, entries and work items written"),
        "sparse_attn": dict(bound="mfma", flops=f_attn - f_loc,
                            what="4*d flops per (query, head, key) of the non-local selected "
                                 "blocks", side_bytes=kv_bytes, triples=n_trip, buckets=n_bkt,
                            min_bytes=rows_q * Hq * D * 2 + n_bkt * 2 * 128 * D * 2,
                            min_bytes_what="each query's Q rows once + each selected K/V block "
                                           "once"),
        "combine": dict(bound="hbm",
                        bytes=n_trip * G * (D * 2 + 4) + rows_q * Hq * D * 2 * 2 + rows_q * Hq * 4
                        + rows * K * 4,
                        flops=f_loc,
                        what="partials (bf16 O + fp32 LSE) read, Q read and O written once, "
                             "LSE written; the local block's attention (flops) runs here"),
    }
    if Nq == 1 and cfg.dtype == si.BF16:
        # decode: the K_idx scan and the query-outer attention stream their operands once
        # (no bucketing, partials or combine), so both are bound by HBM
        DI, eb = cfg.idx_dim, (1 if fp8 else 2)
        keys = B * int(torch.clamp((L + 1) * 128, max=cfg.seqlen_kv).sum().item())
        nbl = int((L + 1).max())
        work["index_blockmax"] = dict(
            bound="hbm", bytes=keys * DI * eb + rows * DI * eb + 4 * rows * nbl
            + (4 * B * nbl + 4 * rows if fp8 else 0),
            flops=f_idx, what="K_idx rows of blocks 0..L read once per sequence, Q_idx read, "
                              "block scores written" + (" (E4M3 bytes and their block and row "
                                                         "exponents)" if fp8 else ""))
        work["sparse_attn"] = dict(
            bound="hbm", bytes=n_sel * 2 * 128 * D * 2 + rows_q * Hq * (2 * D * 2 + 4),
            flops=f_attn, what="K and V of each selected block read once per (sequence, "
                               "group), q read, out and LSE written")
        del work["bucketing"], work["combine"]
    return work, f_idx, f_attn, f_loc, n_sel


def load_traffic(cfg):
    """{timer name: bytes per launch} from the counter record of this workload, for kernels
    whose source is unchanged since the counters were taken."""
    path = traffic_file(cfg.name)
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    out = {}
    for frag, (name, files) in KERNEL_FILES.items():
        e = rec.get("kernels", {}).get(frag)
        if e and e.get("source_hash") == source_hash(files):
            out[name] = e["bytes_per_launch"]
    return out


def ingest_counters(fetch_csv, write_csv, workload, commands):
    """Per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs,
    scaled by what the same counters read for the 1 GiB device copy of --copy-calibration,
    written to profiles/hbm_counters_<workload>.json."""
    import csv
    import collections

    def per_dispatch(path, counter):
        """{kernel: {dispatch id: KiB}} (rows of one dispatch summed)."""
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return acc

    fd, wd = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")
    fe = {k: (sum(v.values()), len(v)) for k, v in fd.items()}
    wr = {k: (sum(v.values()), len(v)) for k, v in wd.items()}
    copy = [k for k in fd if "copyBuffer" in k or "copy_kernel" in k]
    gib_kib = float(1 << 20)
    # the largest single copy dispatch is the 1 GiB calibration copy (other copies of
    # the process are small): it reads and writes 1 GiB
    fcopy = max(max(fd[k].values()) for k in copy)
    wcopy = max(max(wd[k].values()) for k in copy if k in wd)
    fs, ws = gib_kib / fcopy, gib_kib / wcopy
    kernels = {}
    for frag, (name, files) in KERNEL_FILES.items():
        hits = [k for k in fe if frag in k]
        if not hits:
            continue
        k = hits[0]
        f, n = fe[k]
        w, _ = wr.get(k, (0.0, n))
        kernels[frag] = {"kernel": k[:120], "timer": name, "dispatches": n,
                         "fetch_kib_raw": f / n, "write_kib_raw": w / n,
                         "read_bytes": f / n * fs * 1024, "write_bytes": w / n * ws * 1024,
                         "bytes_per_launch": (f / n * fs + w / n * ws) * 1024,
                         "source_hash": source_hash(files)}
    rec = {"workload": workload, "fetch_scale": fs, "write_scale": ws,
           "calibration": "1 GiB device copy in the same process (bench.py --copy-calibration)",
           "commands": commands, "kernels": kernels}
    json.dump(rec, open(traffic_file(workload), "w"), indent=1)
    print(json.dumps({k: round(v["bytes_per_launch"] / 1e9, 3) for k, v in kernels.items()}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="skewed_n131072 by default (train_b2_n32768 with --dense)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kl", action="store_true",
                    help="add msa_kl_align (with the index-logit gradient) to the step; "
                         "a training-side measurement, not the headline line")
    ap.add_argument("--bwd", action="store_true",
                    help="add msa_attn_bwd (dq, dk, dv for a seeded dout) to the step; "
                         "a training-side measurement, not the headline line")
    ap.add_argument("--dense", action="store_true",
                    help="time the warm-up stage instead (dense LSE, KL on the full causal "
                         "context with block masses, selection and block / score recall)")
    ap.add_argument("--fp8", action="store_true",
                    help="select with the FP8 (E4M3) index path: Q_idx quantized every step, "
                         "K_idx every step for prefill and once (as a cache holds it) for "
                         "decode; reports the churn against the bf16 selection")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the per-kernel HBM counter record of --workload from two "
                         "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--commands", nargs="*", default=[],
                    help="the profiler commands recorded with --ingest-counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the MSA layer on a single "
              "MI355X (sharding is a design, not code); --gpus must be 1.", file=sys.stderr)
        sys.exit(2)
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, args.workload or "skewed_n131072", args.commands)
        return

    import torch

    import learned_kv_block_amd as msa
    import seeded_inputs as si

    # the measurement build: the same kernels, with HIP events recorded around each launch
    msa.use_timed_build()
    if args.dense:
        dense_main(args)
        return

    cfg = si.CONFIGS[args.workload or "skewed_n131072"]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    names_in = ("q", "k", "v", "q_idx", "k_idx") + (("dout",) if args.bwd else ())
    x = {n: si.device_tensor(cfg, n, dev) for n in names_in}
    sh_sel = msa.shape_for(x["q_idx"], x["k_idx"], cfg.topk, cfg.q_start, cfg.num_q_heads,
                           cfg.head_dim)
    ws_sel = torch.empty(msa.workspace_size(sh_sel, msa.MSA_OP_SELECT), dtype=torch.uint8,
                         device=dev)
    ws_attn = torch.empty(msa.workspace_size(sh_sel, msa.MSA_OP_ATTN), dtype=torch.uint8,
                          device=dev)
    out = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device=dev)
    ws_kl = (torch.empty(msa.workspace_size(sh_sel, msa.MSA_OP_KL), dtype=torch.uint8,
                         device=dev) if args.kl else None)
    ws_bwd = (torch.empty(msa.workspace_size(sh_sel, msa.MSA_OP_ATTN_BWD), dtype=torch.uint8,
                          device=dev) if args.bwd else None)
    ws_ibwd = (torch.empty(msa.workspace_size(sh_sel, msa.MSA_OP_IDX_BWD), dtype=torch.uint8,
                           device=dev) if args.bwd and args.kl else None)

    decode = cfg.seqlen_q == 1
    kz = (msa.msa_index_quantize_fp8(None, x["k_idx"], q_start=cfg.q_start)
          if args.fp8 and decode else None)

    def select():
        if not args.fp8:
            return msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start,
                                  num_q_heads=cfg.num_q_heads, head_dim=cfg.head_dim,
                                  workspace=ws_sel)
        if decode:  # the cache holds K_idx in FP8; only the new query rows are quantized
            qz = msa.msa_index_quantize_fp8(x["q_idx"], None, seqlen_kv=cfg.seqlen_kv,
                                            q_start=cfg.q_start)
            qz.update(kz)
        else:
            qz = msa.msa_index_quantize_fp8(x["q_idx"], x["k_idx"], q_start=cfg.q_start)
        return msa.msa_select_fp8(qz["q8"], qz["q_exp"], qz["k8"], qz["k_exp"], cfg.topk,
                                  q_start=cfg.q_start, num_q_heads=cfg.num_q_heads,
                                  head_dim=cfg.head_dim, workspace=ws_sel)

    def step():
        sel = select()
        msa.msa_attn_fwd(x["q"], x["k"], x["v"], sel["ids"], q_start=cfg.q_start,
                         idx_dim=cfg.idx_dim, workspace=ws_attn, out=out, lse=lse)
        if args.kl:
            kl = msa.msa_kl_align(x["q"], x["k"], x["q_idx"], x["k_idx"], sel["ids"], lse,
                                  q_start=cfg.q_start, want_dlogits=True, workspace=ws_kl)
        if args.bwd:
            msa.msa_attn_bwd(x["q"], x["k"], x["v"], sel["ids"], out, lse, x["dout"],
                             q_start=cfg.q_start, idx_dim=cfg.idx_dim, workspace=ws_bwd)
            if args.kl:  # the KL gradient into the index projections
                msa.msa_idx_bwd(x["q_idx"], x["k_idx"], sel["ids"], kl["dlogits"],
                                1.0 / (cfg.batch * cfg.seqlen_q * cfg.num_kv_heads),
                                q_start=cfg.q_start, num_q_heads=cfg.num_q_heads,
                                head_dim=cfg.head_dim, workspace=ws_ibwd)
        return sel["ids"]

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    ids = None
    for _ in range(args.warmup):
        ids = step()
    torch.cuda.synchronize()
    if ids is None:
        ids = step()
        torch.cuda.synchronize()
    work, f_idx, f_attn, f_loc, n_sel = step_work(cfg, ids, fp8=args.fp8)

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    # every kernel of the step is timed by HIP events on its launch stream
    with msa.KernelTimer(None, max_launches=max(64, args.steps * 64)) as kt:
        t0 = time.perf_counter()
        ev[0].record()
        for j in range(args.steps):
            step()
            ev[j + 1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    step_ms = sorted(ev[j].elapsed_time(ev[j + 1]) for j in range(args.steps))
    ms_per_step = 1e3 * elapsed / max(1, args.steps)
    tokens = cfg.batch * cfg.seqlen_q
    value = tokens * args.steps / elapsed

    per = kt.per_kernel  # name -> (total ms, launches)
    kernel_ms = {n: round(v[0] / args.steps, 4) for n, v in per.items()}  # per step
    launches = {n: v[1] for n, v in per.items()}
    bucket_names = ("bucket_hist", "bucket_scan", "bucket_scatter", "work_items")
    traffic = {} if args.fp8 else load_traffic(cfg)
    kernels = {}
    for name, w in work.items():
        if name == "bucketing":
            ms = sum(kernel_ms.get(n, 0.0) for n in bucket_names)
            nl = max([launches.get(n, 0) for n in bucket_names] + [0])
            cbytes = (sum(traffic[n] for n in bucket_names if n in traffic)
                      if all(n in traffic for n in ("bucket_hist", "bucket_scatter", "work_items"))
                      else None)
        else:
            src = "index_fp8" if (name == "index_blockmax" and args.fp8) else name
            ms = kernel_ms.get(src, 0.0)
            nl = launches.get(src, 0)
            cbytes = traffic.get(src)
        if ms <= 0.0:
            continue
        e = {"ms": ms, "launches_per_step": nl / max(1, args.steps), "bound": w["bound"],
             "what": w["what"]}
        e["timer"] = src if name != "bucketing" else "bucket_*"
        if w["bound"] == "mfma":
            peak = PEAK_FP8 if (name == "index_blockmax" and args.fp8) else PEAK_BF16
            e.update(flops=w["flops"], achieved_tflops=w["flops"] / (ms * 1e-3) / 1e12,
                     peak_tflops=peak / 1e12, frac=w["flops"] / (ms * 1e-3) / peak)
        else:
            e.update(bytes=w["bytes"], achieved_gbs=w["bytes"] / (ms * 1e-3) / 1e9,
                     peak_gbs=PEAK_HBM / 1e9, frac=w["bytes"] / (ms * 1e-3) / PEAK_HBM)
            if "flops" in w:
                e["flops"] = w["flops"]
        for extra in ("side_bytes", "triples", "buckets", "min_bytes", "min_bytes_what"):
            if extra in w:
                e[extra] = w[extra]
        # counter bytes are per launch; the work fields above are per step
        e["counter_bytes"] = cbytes
        if cbytes is not None and "min_bytes" in w:
            e["counter_over_min_bytes"] = cbytes * e["launches_per_step"] / w["min_bytes"]
        kernels[name] = e
    for n, ms in kernel_ms.items():  # training-side kernels and anything not tabled above
        if n not in kernels and n not in bucket_names and not (n == "index_fp8" and args.fp8):
            kernels[n] = {"ms": ms, "launches_per_step": launches[n] / max(1, args.steps)}
    # the headline roofline is that of the step's dominant tabled kernel
    dom = max((n for n in kernels if "bound" in kernels[n]), key=lambda n: kernels[n]["ms"])
    d = kernels[dom]
    # the roofline is per launch: a kernel that runs several times a step (the
    # attention of a windowed prefill) reports its work and time per launch
    lps = max(1e-9, d["launches_per_step"])
    if d["bound"] == "mfma":
        roofline = {"bound": "mfma", "kernel": dom, "achieved": d["achieved_tflops"],
                    "peak": d["peak_tflops"], "unit": "TFLOP/s", "frac": d["frac"],
                    "traffic": d["counter_bytes"], "avg_ms": d["ms"] / lps,
                    "launches": launches.get(d["timer"], 0), "flops_per_launch": d["flops"] / lps}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": d["achieved_gbs"],
                    "peak": d["peak_gbs"], "unit": "GB/s", "frac": d["frac"],
                    "traffic": d["counter_bytes"], "avg_ms": d["ms"] / lps,
                    "launches": launches.get(d["timer"], 0), "bytes_per_launch": d["bytes"] / lps}
    for extra in ("side_bytes", "min_bytes"):
        if extra in d:
            roofline[extra] = d[extra] / lps
    if "counter_over_min_bytes" in d:
        roofline["counter_over_min_bytes"] = d["counter_over_min_bytes"]
    line = {
        "metric": "MSA-layer prefill query-tokens/s at N=128K (1 GPU) + % bf16 MFMA peak",
        "value": value,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seqlen_kv,
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "idx_dim": cfg.idx_dim,
                   "block_size": cfg.block_size, "topk": cfg.topk, "parallelism": "none"},
        "ms_per_step_median": step_ms[len(step_ms) // 2] if step_ms else None,
        "effective_flops_per_step": f_idx + f_attn,
        "tile_flops_per_step": sum(tile_flops(cfg, ids)),
        "index_flops_per_step": f_idx,
        "attn_flops_per_step": f_attn,
        "attn_local_flops_per_step": f_loc,
        "mfma_frac_effective": (f_idx + f_attn) / (ms_per_step * 1e-3) / PEAK_BF16,
        "kernels": kernels,
        "roofline": roofline,
    }
    if decode:
        line["metric"] = "MSA decode query-tokens/s (one query per sequence)"
    elif cfg.name != "skewed_n131072":
        line["metric"] = f"MSA-layer prefill query-tokens/s ({cfg.name}, 1 GPU)"
    if args.fp8:
        line["metric"] = ("MSA-layer prefill query-tokens/s with the FP8 (E4M3) index branch"
                          if not decode else "MSA decode query-tokens/s with the FP8 index branch")
        line["config"]["index_dtype"] = "fp8_e4m3"
        # churn of the FP8 selection against the bf16 one on the same inputs
        s16 = msa.msa_select(x["q_idx"], x["k_idx"], cfg.topk, q_start=cfg.q_start,
                             want_margin=True, num_q_heads=cfg.num_q_heads,
                             head_dim=cfg.head_dim)
        ids8 = select()["ids"]
        changed = (s16["ids"] != ids8).any(dim=-1)
        small = torch.isfinite(s16["margin"]) & (s16["margin"] < 0.03)
        big = torch.isfinite(s16["margin"]) & (s16["margin"] >= 0.1)
        line["fp8_churn"] = {
            "changed_share": float(changed.float().mean()),
            "changed_share_margin_lt_0.03":
                float(changed[small].float().mean()) if bool(small.any()) else 0.0,
            "changed_share_margin_ge_0.1":
                float(changed[big].float().mean()) if bool(big.any()) else 0.0}
        del s16, ids8, changed, small, big
    if args.kl:
        line["metric"] = "MSA-layer training step (select + attention + KL align) query-tokens/s"
        line["config"]["kl"] = True
    if args.bwd:
        parts = ("select + attention" + (" + KL align" if args.kl else "") + " + attention backward" +
                 (" + index backward" if args.kl else ""))
        line["metric"] = f"MSA-layer training step ({parts}) query-tokens/s"
        line["config"]["bwd"] = True
        # recomputed S and P, dP, dV, dK, dQ: five products of the forward's two,
        # on every selected (query, head, key) including the local blocks
        line["attn_bwd_flops_per_step"] = 2.5 * f_attn
        if "attn_bwd" in kernel_ms:
            line["attn_bwd_mfma_frac"] = 2.5 * f_attn / (kernel_ms["attn_bwd"] * 1e-3) / PEAK_BF16
    print(f"[bench] kernels {kernel_ms}", file=sys.stderr, flush=True)
    del x, ws_sel, ws_attn, ws_kl, ws_bwd, ws_ibwd, out, lse, kz
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
