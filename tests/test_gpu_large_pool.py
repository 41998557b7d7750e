"""Pools larger than 4 GiB: a batch's pages moved to ids whose byte offsets
exceed 32 bits (the largest pool sizes an MI355X's 288 GB hold).  Every
kernel that reads or writes the pool must give exactly what it gives on the
same batch with its pages at small ids (outputs are bit-identical under a
change of physical page ids), and attention must still match the oracle.
One 5 GiB buffer per pool serves every shape (viewed as [pages, Hkv, 16, d])."""
import numpy as np
import pytest
import torch

import oracle as ORACLE
import paged_kv_cache_02_amd as pa
import workloads as W
from helpers import compare, device_batch, oracle_run, to_torch

pytestmark = pytest.mark.gpu

POOL_BYTES = 5 << 30
FOUR_GIB = 1 << 32


@pytest.fixture(scope="module")
def big_pools():
    k = torch.empty(POOL_BYTES, dtype=torch.uint8, device="cuda")
    v = torch.empty(POOL_BYTES, dtype=torch.uint8, device="cuda")
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def view_pool(buf, b):
    tdt = torch.bfloat16 if b.dtype == W.BF16 else torch.float32
    _, Hkv, P, d = b.k_pool.shape
    per_page = Hkv * P * d * (2 if b.dtype == W.BF16 else 4)
    return buf.view(tdt)[: (POOL_BYTES // per_page) * Hkv * P * d].view(-1, Hkv, P, d), per_page


def relocate(b, big_pools, seed):
    """Device batch whose pages sit at ids past the 4 GiB byte offset of a
    5 GiB pool; returns (dev dict, the ids used, the relocated table)."""
    kb, per_page = view_pool(big_pools[0], b)
    vb, _ = view_pool(big_pools[1], b)
    n = b.k_pool.shape[0]
    total = kb.shape[0]
    first_high = FOUR_GIB // per_page + 1
    assert total - first_high >= n
    rng = np.random.default_rng(seed)
    ids = (first_high + rng.permutation(total - first_high)[:n]).astype(np.int64)
    assert ids.min() * per_page > FOUR_GIB
    idx = torch.from_numpy(ids).cuda()
    kb.index_copy_(0, idx, to_torch(b.k_pool, b.dtype))
    vb.index_copy_(0, idx, to_torch(b.v_pool, b.dtype))
    pt = np.where(b.page_table >= 0, ids[np.maximum(b.page_table, 0)], -1).astype(np.int32)
    dev = device_batch(b)
    dev["k_pool"], dev["v_pool"] = kb, vb
    dev["page_table"] = torch.from_numpy(pt).cuda()
    return dev, ids, pt


def decode_batch(seed, d, dtype, Hq=32, Hkv=8):
    rng = np.random.default_rng(seed)
    L = rng.integers(1, 3000, size=12).astype(np.int32)
    return W.make_batch(f"large pool decode {seed}", seed, L, L - 1, Hq, Hkv, d, 16, dtype)


@pytest.mark.parametrize("d,dtype,Hq,Hkv", [(128, W.BF16, 32, 8), (64, W.BF16, 32, 8), (64, W.F32, 8, 2)])
def test_decode_past_4gib(big_pools, d, dtype, Hq, Hkv):
    b = decode_batch(200 + d, d, dtype, Hq, Hkv)
    print(f"case large pool decode d={d} {dtype}", flush=True)
    small = device_batch(b)
    ref_out, ref_lse = pa.pa_decode(small["q"], small["k_pool"], small["v_pool"], small["page_table"],
                                    small["seq_lens"], small["q_offsets"], b.scale, max_seq_len=b.max_seq_len)
    dev, _, _ = relocate(b, big_pools, 1)
    desc = pa.make_desc(dev["q"], dev["k_pool"], dev["page_table"], dev["seq_lens"], b.max_seq_len)
    assert pa.pa_plan(desc)["path"] == "decode_balanced"
    out, lse = pa.pa_decode(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"], dev["seq_lens"],
                            dev["q_offsets"], b.scale, desc=desc)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label=f"large pool decode d={d} {dtype}")
    # equal splits, through the same relocated pages
    out_s, lse_s, _ = pa.pa_split_merge(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                        dev["seq_lens"], dev["q_offsets"], b.scale, 4, desc=desc)
    torch.cuda.synchronize()
    compare(b, out_s, lse_s, ro, rl, label=f"large pool split S=4 d={d} {dtype}")
    # direct (non-flash) paged attention, scores stored in its workspace
    out_d, lse_d = pa.pa_decode_direct(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                       dev["seq_lens"], b.scale, desc=desc)
    torch.cuda.synchronize()
    compare(b, out_d, lse_d, ro, rl, label=f"large pool direct d={d} {dtype}")


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_and_mixed_past_4gib(big_pools, d):
    lens = np.array([700, 300, 129, 1], np.int32)
    offs = np.array([200, 0, 64, 0], np.int32)
    b = W.make_batch(f"large pool prefill {d}", 300 + d, lens, offs, 32, 8, d, 16, W.BF16)
    print(f"case large pool prefill d={d}", flush=True)
    small = device_batch(b)
    ref_out, ref_lse = pa.pa_prefill_chunk(small["q"], small["k_pool"], small["v_pool"],
                                           small["page_table"], small["seq_lens"], small["q_offsets"],
                                           b.scale, max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
    dev, _, _ = relocate(b, big_pools, 2)
    out, lse = pa.pa_prefill_chunk(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                   dev["seq_lens"], dev["q_offsets"], b.scale, max_seq_len=b.max_seq_len,
                                   max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label=f"large pool prefill d={d}")
    out_m, lse_m = pa.pa_mixed_attention(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                         dev["seq_lens"], dev["q_offsets"], b.scale,
                                         max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    compare(b, out_m, lse_m, ro, rl, label=f"large pool mixed d={d}")


def test_append_copy_and_gather_past_4gib(big_pools):
    lens = np.array([37, 300, 129], np.int32)
    offs = np.array([0, 170, 128], np.int32)
    Hkv, d = 8, 128
    b = W.make_batch("large pool append", 400, lens, offs, Hkv, Hkv, d, 16, W.BF16, pool_factor=1.5)
    rng = np.random.default_rng(401)
    rows = int(b.total_q)
    kn = W.f32_to_bf16_bits(rng.standard_normal((rows, Hkv, d)).astype(np.float32))
    vn = W.f32_to_bf16_bits(rng.standard_normal((rows, Hkv, d)).astype(np.float32))
    print("case large pool append, copy, gather", flush=True)
    dev, ids, pt = relocate(b, big_pools, 3)
    pa.pa_append_kv(to_torch(kn, W.BF16), to_torch(vn, W.BF16), dev["k_pool"], dev["v_pool"],
                    dev["page_table"], dev["seq_lens"], dev["q_offsets"], max_seq_len=b.max_seq_len,
                    max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    ek, ev = ORACLE.append_kv(b.k_pool, b.v_pool, b.page_table, b.seq_lens, b.q_offsets, kn, vn)
    idx = torch.from_numpy(ids).cuda()
    got_k = dev["k_pool"].index_select(0, idx).cpu().view(torch.int16).numpy().view(np.uint16)
    got_v = dev["v_pool"].index_select(0, idx).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_k, ek) and np.array_equal(got_v, ev)
    # the gather through the relocated table equals the oracle's gather of the compact pool
    for r in range(len(lens)):
        k, v = pa.pa_gather_kv(dev["k_pool"], dev["v_pool"], dev["page_table"], r, int(lens[r]))
        gk, gv = ORACLE.gather(ek, ev, b.page_table[r], int(lens[r]))
        assert np.array_equal(k.cpu().view(torch.int16).numpy().view(np.uint16), gk)
        assert np.array_equal(v.cpu().view(torch.int16).numpy().view(np.uint16), gv)
    # whole-page copies from past 4 GiB down to low ids and back up
    low = np.array([5, 9], np.int32)
    src = np.array([ids[0], ids[1]], np.int32)
    desc = pa.make_desc(dev["q"], dev["k_pool"], dev["page_table"], dev["seq_lens"], b.max_seq_len,
                        b.max_q_len, dev["q_offsets"])
    pa.pa_copy_pages(dev["k_pool"], dev["v_pool"], torch.from_numpy(src).cuda(), torch.from_numpy(low).cuda(),
                     desc=desc)
    up = np.array([ids[2], ids[3]], np.int32)
    pa.pa_copy_pages(dev["k_pool"], dev["v_pool"], torch.from_numpy(low).cuda(), torch.from_numpy(up).cuda(),
                     desc=desc)
    torch.cuda.synchronize()
    for s, t in ((0, 2), (1, 3)):
        a = dev["k_pool"][int(ids[s])].cpu().view(torch.int16).numpy()
        c = dev["k_pool"][int(ids[t])].cpu().view(torch.int16).numpy()
        assert np.array_equal(a, c)
        a = dev["v_pool"][int(ids[s])].cpu().view(torch.int16).numpy()
        c = dev["v_pool"][int(ids[t])].cpu().view(torch.int16).numpy()
        assert np.array_equal(a, c)
