"""Seeded random parity sweep: each case draws a route (guard-routed decode,
equal-split decode, chunked prefill, the single mixed launch), a head dim,
a KV-head count, a head ratio, a batch of context lengths and chunk offsets,
and a pool layout (permuted with spare pages, or exactly the needed pages
grown round-robin), and compares every output row and lse with the oracle.
The draws stay inside each entry point's contract; the sizes keep the
oracle to about a second per case."""
import numpy as np
import pytest
import torch

import paged_kv_cache_02_amd as pa
import workloads as W
from helpers import compare, device_batch, oracle_run

pytestmark = pytest.mark.gpu

ROUTES = ("decode", "split", "prefill", "mixed")
CASES = 64


def draw(case):
    rng = np.random.default_rng(20_000 + case)
    route = ROUTES[case % len(ROUTES)]
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    dtype = W.BF16
    if route in ("decode", "split"):
        if rng.random() < 0.3:
            dtype = W.F32
        G = int(rng.integers(1, (8 if dtype == W.F32 else 16) + 1))
        B = int(rng.integers(1, 120))
        L = rng.integers(1, 4000, size=B).astype(np.int32)
        o = L - 1
    elif route == "prefill":
        G = int(rng.integers(1, 13))
        B = int(rng.integers(1, 6))
        o = rng.integers(0, 2000, size=B).astype(np.int32)
        n = rng.integers(1, 200, size=B).astype(np.int32)
        L = o + n
    else:
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(2, 17))
        n = np.where(rng.random(B) < 0.5, 1, rng.integers(2, 80, size=B)).astype(np.int32)
        L = rng.integers(1, 1500, size=B).astype(np.int32) + n
        o = L - n
    Hkv = min(Hkv, max(1, 64 // G))   # at most 64 query heads keeps the oracle quick
    pool = "permuted" if rng.random() < 0.7 else "interleaved"
    b = W.make_batch(f"sweep{case}", 30_000 + case, L, o, G * Hkv, Hkv, d, 16, dtype, pool=pool,
                     pool_factor=float(rng.uniform(1.0, 2.0)), rng=rng)
    S = int(rng.integers(1, 24))
    return route, b, S


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(case):
    route, b, S = draw(case)
    G = b.num_q_heads // b.num_kv_heads
    print(f"case sweep {case}: {route} B={b.num_seqs} Hq={b.num_q_heads} Hkv={b.num_kv_heads} "
          f"d={b.head_dim} {b.dtype} G={G} S={S} max L={int(b.seq_lens.max())}", flush=True)
    dev = device_batch(b)
    args = (dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"], dev["seq_lens"], dev["q_offsets"],
            b.scale)
    if route == "decode":
        out, lse = pa.pa_decode(*args, max_seq_len=b.max_seq_len)
    elif route == "split":
        out, lse, _ = pa.pa_split_merge(*args, S, max_seq_len=b.max_seq_len)
    elif route == "prefill":
        out, lse = pa.pa_prefill_chunk(*args, max_seq_len=b.max_seq_len, max_q_len=b.max_q_len,
                                       split=bool(case % 8 < 4))
    else:
        out, lse = pa.pa_mixed_attention(*args, max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label=f"sweep {case} {route}")
