"""GPU parity of the two measurement baselines against the oracle: the fused
decode kernel over a dense (unpaged) cache, and direct paged attention
without the flash fusion (scores stored, softmax, then values)."""
import numpy as np
import pytest
import torch

import oracle as ORACLE
import paged_kv_cache_02_amd as pa
import workloads as W
from helpers import compare, device_batch, oracle_run, to_torch

pytestmark = pytest.mark.gpu


def ragged(seed, lens, Hq, Hkv, d, dtype=W.BF16, **kw):
    L = np.array(lens, np.int32)
    return W.make_batch(f"base{seed}", seed, L, L - 1, Hq, Hkv, d, 16, dtype, **kw)


def dense_cache(b: W.PagedBatch):
    """The batch's keys and values as dense [B, Hkv, MP * P, d] caches (the
    oracle's gather of each request, zero past seq_len)."""
    B, MP, P = len(b.seq_lens), b.page_table.shape[1], b.page_size
    shape = (B, b.num_kv_heads, MP * P, b.head_dim)
    kd = np.zeros(shape, b.k_pool.dtype)
    vd = np.zeros(shape, b.v_pool.dtype)
    for r in range(B):
        L = int(b.seq_lens[r])
        K, V = ORACLE.gather(b.k_pool, b.v_pool, b.page_table[r], L)   # [L, Hkv, d], raw storage
        kd[r, :, :L] = np.transpose(K, (1, 0, 2))
        vd[r, :, :L] = np.transpose(V, (1, 0, 2))
    return kd, vd


CASES = [
    dict(seed=1, lens=[37, 100], Hq=4, Hkv=2, d=64, dtype=W.F32),
    dict(seed=2, lens=[1, 16, 17, 300, 1000], Hq=32, Hkv=8, d=128, dtype=W.BF16),
    dict(seed=3, lens=[513, 2049, 90], Hq=16, Hkv=8, d=128, dtype=W.BF16),
    dict(seed=4, lens=[700, 33], Hq=8, Hkv=8, d=64, dtype=W.BF16),
    dict(seed=5, lens=[260, 5], Hq=16, Hkv=2, d=128, dtype=W.BF16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_dense_cache_decode_matches_oracle(case):
    b = ragged(case["seed"], case["lens"], case["Hq"], case["Hkv"], case["d"], case["dtype"])
    dev = device_batch(b)
    kd, vd = dense_cache(b)
    desc = pa.make_desc(dev["q"], dev["k_pool"], dev["page_table"], dev["seq_lens"], b.max_seq_len)
    print(f"case dense seed={case['seed']} lens={case['lens']}", flush=True)
    out, lse = pa.pa_decode_dense(dev["q"], to_torch(kd, b.dtype), to_torch(vd, b.dtype), dev["seq_lens"],
                                  b.scale, desc=desc)
    torch.cuda.synchronize()
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label=f"dense {case['seed']}")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c['seed']}")
def test_direct_paged_decode_matches_oracle(case):
    b = ragged(case["seed"], case["lens"], case["Hq"], case["Hkv"], case["d"], case["dtype"])
    dev = device_batch(b)
    desc = pa.make_desc(dev["q"], dev["k_pool"], dev["page_table"], dev["seq_lens"], b.max_seq_len)
    print(f"case direct seed={case['seed']} lens={case['lens']}", flush=True)
    out, lse = pa.pa_decode_direct(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                   dev["seq_lens"], b.scale, desc=desc)
    torch.cuda.synchronize()
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label=f"direct {case['seed']}")


def test_baselines_on_the_qwen3_4b_decode_shapes():
    b = W.make_config("qwen3_4b_decode")
    dev = device_batch(b)
    desc = pa.make_desc(dev["q"], dev["k_pool"], dev["page_table"], dev["seq_lens"], b.max_seq_len)
    rows = np.random.default_rng(0).choice(len(b.seq_lens), 6, replace=False)
    ro, rl = oracle_run(b, requests=rows)
    out, lse = pa.pa_decode_direct(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                   dev["seq_lens"], b.scale, desc=desc)
    torch.cuda.synchronize()
    compare(b, out, lse, ro, rl, rows=rows, label="direct qwen3-4b")
    kd, vd = dense_cache(b)
    out, lse = pa.pa_decode_dense(dev["q"], to_torch(kd, b.dtype), to_torch(vd, b.dtype), dev["seq_lens"],
                                  b.scale, desc=desc)
    torch.cuda.synchronize()
    compare(b, out, lse, ro, rl, rows=rows, label="dense qwen3-4b")
