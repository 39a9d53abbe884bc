"""msa_attn_fwd_noalloc (the allocation-free variant of msa_attn_fwd) through the C ABI.

Its kernels and launch sequence are those of msa_attn_fwd; only the workspace differs (the
library's fixed device scratch instead of a caller buffer). So on the same inputs and ids
its outputs must equal msa_attn_fwd's bit for bit, also on a second call with a smaller
input that finds the first call's data still in the scratch.
"""
import pytest
import torch

import seeded_inputs as si
from tests import parity

pytestmark = pytest.mark.gpu


def _case(name, **kw):
    return si.CONFIGS["decode_b64_n131072"].replace(name=name, seed=41, **kw)


# largest first, then smaller inputs: the scratch keeps the previous call's contents
CASES = [
    _case("decode_b16_n8192", batch=16, seqlen_kv=8192, q_start=8191),
    _case("decode_b4_n3000", batch=4, seqlen_kv=3000, q_start=2999, topk=6),
    si.CONFIGS["tiny_f32_n1024"],
]


def test_noalloc_equals_attn_fwd_on_consecutive_calls():
    import learned_kv_block_amd as msa
    for cfg in CASES:
        print(f"[noalloc] {cfg.name}", flush=True)
        x = parity.gpu_inputs(cfg)
        res = parity.run_gpu(cfg, x)  # msa_select + msa_attn_fwd with its own workspace
        out = torch.full_like(res["out"], float("nan"))
        lse = torch.full_like(res["lse"], float("nan"))
        msa.msa_attn_fwd_noalloc(x["q"], x["k"], x["v"], res["ids"], out, lse,
                                 q_start=cfg.q_start, idx_dim=cfg.idx_dim)
        torch.cuda.synchronize()
        assert torch.equal(out, res["out"]), cfg.name
        assert torch.equal(lse, res["lse"]), cfg.name
        # the shared outputs also meet the oracle on every row
        parity.check_all(cfg, dict(res, out=out, lse=lse))
        del x, res, out, lse
        torch.cuda.empty_cache()


def test_noalloc_rejects_workloads_beyond_the_scratch():
    import learned_kv_block_amd as msa
    cfg = si.CONFIGS["main_n8192"]
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 8192, 64, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 8192, 4, 128), dtype=torch.bfloat16, device=dev)
    ids = torch.zeros((1, 8192, 4, 16), dtype=torch.int32, device=dev)
    lse = torch.zeros((1, 8192, 64), dtype=torch.float32, device=dev)
    with pytest.raises(msa.MsaError) as e:
        msa.msa_attn_fwd_noalloc(q, k, k, ids, torch.empty_like(q), lse, q_start=cfg.q_start)
    assert e.value.status == msa.MSA_ERR_SCRATCH
