"""pa_decode_noalloc (the decode entry point that allocates nothing and runs
on the library's fixed device scratch) against pa_decode, through the C ABI:
two calls in a row, the second with a smaller batch, each bit-identical to
pa_decode on the same inputs and within the bar of the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_02_amd as pa
import workloads as W
from helpers import compare, device_batch, oracle_run

pytestmark = pytest.mark.gpu


def noalloc_vs_decode(b, rows):
    dev = device_batch(b)
    desc = pa.make_desc(dev["q"], dev["k_pool"], dev["page_table"], dev["seq_lens"], b.max_seq_len)
    plan = pa.pa_plan(desc)
    print(f"case noalloc {b.name} plan={plan}", flush=True)
    assert 0 < plan["workspace_bytes"] <= pa.NOALLOC_SCRATCH_BYTES
    ref, ref_lse = pa.pa_decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                dev["seq_lens"], dev["q_offsets"], b.scale, desc=desc)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    pa.pa_decode_noalloc(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                         dev["seq_lens"], dev["q_offsets"], b.scale, out=out, lse=lse, desc=desc)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    ro, rl = oracle_run(b, requests=rows)
    compare(b, out, lse, ro, rl, rows=rows, label=f"noalloc {b.name}")


def test_noalloc_two_calls_second_smaller():
    # a full Qwen3-4B-shaped batch (page-balanced route, 3.2 MB of scratch),
    # then the smaller Qwen3-0.6B-shaped batch (same route, 1.3 MB) on the
    # same device scratch, which still holds the first call's partials
    big = W.make_config("qwen3_4b_decode")
    noalloc_vs_decode(big, rows=[0, 17, 63])
    small = W.make_config("qwen3_0p6b_decode")
    noalloc_vs_decode(small, rows=[0, 5, 31])


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    # 2048 requests at 64 query heads and d = 128 need about 72 MB of
    # partials: refused before anything is launched
    d = pa.pa_desc(2048, 64, 8, 128, 16, 1 << 20, 512, 2048, 8192, 1, pa.PA_BF16)
    need = pa.pa_plan(d)["workspace_bytes"]
    assert need > pa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(2048, 64, 128, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(16, 8, 16, 128, dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros(2048, 512, dtype=torch.int32, device="cuda")
    sl = torch.ones(2048, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(2048, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_noalloc(q, pool, pool, pt, sl, sl, 0.125, out=out, lse=lse, desc=d)
    assert e.value.code == pa.PA_ERR_WORKSPACE
