"""GPU parity of the KV append (pa_append_kv) against the oracle's append,
byte for byte, and an end-to-end serving sequence: pages from the host
allocator, prefill chunks and decode tokens appended step by step, attention
checked against the oracle after every step."""
import numpy as np
import pytest
import torch

import oracle as ORACLE
import paged_kv_cache_02_amd as pa
import workloads as W
from helpers import compare, device_batch, oracle_run, to_torch

pytestmark = pytest.mark.gpu


def raw(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host bytes as a numpy array of the same element size."""
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def append_case(seed, lens, offs, Hkv, d, dtype, pool_factor=1.5):
    b = W.make_batch(f"append{seed}", seed, np.array(lens, np.int32), np.array(offs, np.int32),
                     Hkv, Hkv, d, 16, dtype, pool_factor=pool_factor)
    rng = np.random.default_rng(seed + 1000)
    rows = int(b.total_q)
    if dtype == W.BF16:
        kn = W.f32_to_bf16_bits(rng.standard_normal((rows, Hkv, d)).astype(np.float32))
        vn = W.f32_to_bf16_bits(rng.standard_normal((rows, Hkv, d)).astype(np.float32))
    else:
        kn = rng.standard_normal((rows, Hkv, d)).astype(np.float32)
        vn = rng.standard_normal((rows, Hkv, d)).astype(np.float32)
    return b, kn, vn


@pytest.mark.parametrize("Hkv,d,dtype", [(8, 128, W.BF16), (2, 64, W.BF16), (4, 128, W.F32),
                                         (1, 64, W.F32), (8, 64, W.BF16), (16, 128, W.F32)])
@pytest.mark.parametrize("with_starts", [False, True])
def test_append_matches_oracle_bit_exact(Hkv, d, dtype, with_starts):
    # prompt from 0, chunks crossing pages, one decode token, page-aligned chunk
    lens = [37, 300, 129, 64, 17]
    offs = [0, 170, 128, 32, 16]
    b, kn, vn = append_case(50 + Hkv + d, lens, offs, Hkv, d, dtype)
    print(f"case append Hkv={Hkv} d={d} {dtype} q_starts={with_starts}", flush=True)
    dev = device_batch(b)
    k_new, v_new = to_torch(kn, dtype), to_torch(vn, dtype)
    qs = torch.from_numpy(b.q_row_starts.astype(np.int32)).cuda() if with_starts else None
    pa.pa_append_kv(k_new, v_new, dev["k_pool"], dev["v_pool"], dev["page_table"], dev["seq_lens"],
                    dev["q_offsets"], q_starts=qs, max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    ek, ev = ORACLE.append_kv(b.k_pool, b.v_pool, b.page_table, b.seq_lens, b.q_offsets, kn, vn)
    gk, gv = raw(dev["k_pool"]), raw(dev["v_pool"])
    assert np.array_equal(gk.view(np.uint8), ek.view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), ev.view(np.uint8))


@pytest.mark.parametrize("with_starts", [False, True])
def test_append_skips_rows_whose_page_is_out_of_range(with_starts):
    b, kn, vn = append_case(77, [40, 20], [8, 0], 2, 64, W.BF16)
    print(f"case append bad page ids q_starts={with_starts}", flush=True)
    dev = device_batch(b)
    bad = dev["page_table"].clone()
    bad[0, 1] = b.num_pages + 5          # positions 16..31 of request 0
    bad[1, 0] = -1                       # positions 0..15 of request 1
    before_k, before_v = raw(dev["k_pool"]).copy(), raw(dev["v_pool"]).copy()
    qs = torch.from_numpy(b.q_row_starts.astype(np.int32)).cuda() if with_starts else None
    pa.pa_append_kv(to_torch(kn, W.BF16), to_torch(vn, W.BF16), dev["k_pool"], dev["v_pool"], bad,
                    dev["seq_lens"], dev["q_offsets"], q_starts=qs, max_seq_len=b.max_seq_len,
                    max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    # the oracle on the same table, with the bad rows' pages pointed at a scratch pool row
    tab = b.page_table.copy()
    tab[0, 1] = b.num_pages              # scratch page past the real pool
    tab[1, 0] = b.num_pages
    pad = lambda p: np.concatenate([p, np.zeros((1,) + p.shape[1:], p.dtype)])
    ek, ev = ORACLE.append_kv(pad(before_k), pad(before_v), tab, b.seq_lens, b.q_offsets, kn, vn)
    assert np.array_equal(raw(dev["k_pool"]).view(np.uint8), ek[:-1].view(np.uint8))
    assert np.array_equal(raw(dev["v_pool"]).view(np.uint8), ev[:-1].view(np.uint8))


@pytest.mark.parametrize("with_starts", [False, True])
def test_append_skips_a_request_with_a_negative_offset(with_starts):
    # a negative q_offset breaks the contract (pa_validate_metadata reports
    # it); the kernel must then skip that request rather than write before
    # its first page
    b, kn, vn = append_case(78, [40, 20], [8, 0], 2, 64, W.BF16)
    print(f"case append negative offset q_starts={with_starts}", flush=True)
    dev = device_batch(b)
    before_k, before_v = raw(dev["k_pool"]).copy(), raw(dev["v_pool"]).copy()
    offs = dev["q_offsets"].clone()
    offs[0] = -4                          # request 0 now claims 44 rows
    rows0 = 40 + 4
    rng = np.random.default_rng(5)
    kn2 = np.concatenate([W.f32_to_bf16_bits(rng.standard_normal((rows0, 2, 64)).astype(np.float32)),
                          kn[32:]])
    vn2 = np.concatenate([W.f32_to_bf16_bits(rng.standard_normal((rows0, 2, 64)).astype(np.float32)),
                          vn[32:]])
    # request 0's claimed rows come first, so request 1's rows start at 44
    qs = torch.tensor([0, rows0, rows0 + 20], dtype=torch.int32, device="cuda") if with_starts else None
    pa.pa_append_kv(to_torch(kn2, W.BF16), to_torch(vn2, W.BF16), dev["k_pool"], dev["v_pool"],
                    dev["page_table"], dev["seq_lens"], offs, q_starts=qs, max_seq_len=b.max_seq_len,
                    max_q_len=b.max_seq_len)   # a valid host bound the device offsets break
    torch.cuda.synchronize()
    # expected: request 1 appended, request 0 and everything else untouched
    ek, ev = ORACLE.append_kv(before_k, before_v, b.page_table[1:], b.seq_lens[1:], b.q_offsets[1:],
                              kn[32:], vn[32:])
    assert np.array_equal(raw(dev["k_pool"]).view(np.uint8), ek.view(np.uint8))
    assert np.array_equal(raw(dev["v_pool"]).view(np.uint8), ev.view(np.uint8))


def test_append_with_an_empty_request_between_others():
    # request 2 appends no row this step (q_offsets == seq_lens): the rows
    # after it belong to request 3, on either launch shape
    b, _, _ = append_case(79, [37, 300, 51, 129], [0, 170, 50, 128], 4, 128, W.BF16)
    offs = b.q_offsets.copy()
    offs[2] = b.seq_lens[2]
    n = (b.seq_lens - offs).astype(np.int64)
    rng = np.random.default_rng(80)
    kn = W.f32_to_bf16_bits(rng.standard_normal((int(n.sum()), 4, 128)).astype(np.float32))
    vn = W.f32_to_bf16_bits(rng.standard_normal((int(n.sum()), 4, 128)).astype(np.float32))
    ek, ev = ORACLE.append_kv(b.k_pool, b.v_pool, b.page_table, b.seq_lens, offs, kn, vn)
    for with_starts in (False, True):
        print(f"case append empty request q_starts={with_starts}", flush=True)
        dev = device_batch(b)
        qs = (torch.from_numpy(np.concatenate([[0], np.cumsum(n)]).astype(np.int32)).cuda()
              if with_starts else None)
        pa.pa_append_kv(to_torch(kn, W.BF16), to_torch(vn, W.BF16), dev["k_pool"], dev["v_pool"],
                        dev["page_table"], dev["seq_lens"], torch.from_numpy(offs).cuda(), q_starts=qs,
                        max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
        torch.cuda.synchronize()
        assert np.array_equal(raw(dev["k_pool"]).view(np.uint8), ek.view(np.uint8))
        assert np.array_equal(raw(dev["v_pool"]).view(np.uint8), ev.view(np.uint8))


@pytest.mark.parametrize("B", [256, 300])
def test_append_many_requests_with_row_starts(B):
    # decode-like steps (one or a few rows per request) with q_starts: up to
    # 256 requests take the launch over the step's rows, more take one
    # workgroup per request
    rng = np.random.default_rng(81 + B)
    L = rng.integers(2, 200, size=B).astype(np.int32)
    n = np.minimum(L, rng.integers(1, 4, size=B)).astype(np.int32)
    b, kn, vn = append_case(82 + B, L, L - n, 2, 64, W.BF16)
    print(f"case append B={B} rows={int(b.total_q)} q_starts=True", flush=True)
    dev = device_batch(b)
    qs = torch.from_numpy(b.q_row_starts.astype(np.int32)).cuda()
    pa.pa_append_kv(to_torch(kn, W.BF16), to_torch(vn, W.BF16), dev["k_pool"], dev["v_pool"],
                    dev["page_table"], dev["seq_lens"], dev["q_offsets"], q_starts=qs,
                    max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    ek, ev = ORACLE.append_kv(b.k_pool, b.v_pool, b.page_table, b.seq_lens, b.q_offsets, kn, vn)
    assert np.array_equal(raw(dev["k_pool"]).view(np.uint8), ek.view(np.uint8))
    assert np.array_equal(raw(dev["v_pool"]).view(np.uint8), ev.view(np.uint8))


def test_serving_sequence_allocator_append_attention():
    """Three requests served for several steps: the host allocator reserves
    pages as sequences grow, pa_append_kv writes each step's K/V, then the
    step's attention (chunked prefill, then decode) is compared with the
    oracle on the same cache; a finished request releases its pages, and a
    new request reuses them."""
    rng = np.random.default_rng(5)
    Hq, Hkv, d, P = 16, 4, 128, 16
    NP, MP = 64, 24
    pool = pa.PagePool(NP)
    k_pool = torch.zeros(NP, Hkv, P, d, dtype=torch.bfloat16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    kp_host = np.zeros((NP, Hkv, P, d), np.uint16)   # the oracle's copy of the pools
    vp_host = np.zeros_like(kp_host)
    table = np.full((3, MP), -1, np.int32)
    lens = np.zeros(3, np.int64)
    prompts = [200, 75, 130]
    chunk = 64
    scale = 1.0 / np.sqrt(d)
    steps = 0
    while steps < 14:
        steps += 1
        # this step's rows: next prompt chunk, or one decode token
        n = np.array([min(chunk, prompts[r] - lens[r]) if lens[r] < prompts[r] else 1
                      for r in range(3)], np.int64)
        offs = lens.copy()
        new = lens + n
        for r in range(3):
            pool.reserve(table[r], int(lens[r]), int(new[r]), P)
        rows = int(n.sum())
        kn = W.f32_to_bf16_bits(rng.standard_normal((rows, Hkv, d)).astype(np.float32))
        vn = W.f32_to_bf16_bits(rng.standard_normal((rows, Hkv, d)).astype(np.float32))
        q = W.f32_to_bf16_bits(rng.standard_normal((rows, Hq, d)).astype(np.float32))
        sl = torch.from_numpy(new.astype(np.int32)).cuda()
        qo = torch.from_numpy(offs.astype(np.int32)).cuda()
        pt = torch.from_numpy(table).cuda()
        pa.pa_append_kv(to_torch(kn, W.BF16), to_torch(vn, W.BF16), k_pool, v_pool, pt, sl, qo,
                        max_seq_len=int(new.max()), max_q_len=int(n.max()))
        kp_host, vp_host = ORACLE.append_kv(kp_host, vp_host, table, new, offs, kn, vn)
        # attention over the updated cache
        qt = to_torch(q, W.BF16)
        if n.max() > 1:
            out, lse = pa.pa_prefill_chunk(qt, k_pool, v_pool, pt, sl, qo, scale,
                                           max_seq_len=int(new.max()), max_q_len=int(n.max()))
        else:
            out, lse = pa.pa_decode(qt, k_pool, v_pool, pt, sl, qo, scale, max_seq_len=int(new.max()))
        torch.cuda.synchronize()
        assert np.array_equal(raw(k_pool).view(np.uint8), kp_host.view(np.uint8))
        b = W.PagedBatch(name=f"serve{steps}", seed=0, q=q, k_pool=kp_host, v_pool=vp_host,
                         page_table=table.copy(), seq_lens=new.astype(np.int32),
                         q_offsets=offs.astype(np.int32), num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=d, page_size=P, scale=scale, dtype=W.BF16)
        ro, rl = oracle_run(b)
        compare(b, out, lse, ro, rl, label=f"serve step {steps}")
        lens = new
        if steps == 9:                      # request 1 finishes; a new one takes its slot
            pool.release(table[1], int(lens[1]), P)
            lens[1] = 0
            prompts[1] = 90
    assert pool.num_free == NP - sum(int((table[r] >= 0).sum()) for r in range(3))


@pytest.mark.parametrize("Hkv,d,dtype", [(8, 128, W.BF16), (2, 64, W.F32)])
def test_copy_pages_matches_oracle_bit_exact(Hkv, d, dtype):
    rng = np.random.default_rng(31)
    NP, P = 40, 16
    if dtype == W.BF16:
        kp = W.f32_to_bf16_bits(rng.standard_normal((NP, Hkv, P, d)).astype(np.float32))
        vp = W.f32_to_bf16_bits(rng.standard_normal((NP, Hkv, P, d)).astype(np.float32))
    else:
        kp = rng.standard_normal((NP, Hkv, P, d)).astype(np.float32)
        vp = rng.standard_normal((NP, Hkv, P, d)).astype(np.float32)
    src = np.array([3, 17, 0, 25, 39, 12, -1, 8], np.int32)
    dst = np.array([30, 1, 22, 5, 36, 12, 9, 99], np.int32)   # a self-copy and two bad pairs
    kt, vt = to_torch(kp, dtype), to_torch(vp, dtype)
    desc = pa.pa_desc(1, Hkv, Hkv, d, P, NP, 4, 1, P, 1, pa.PA_BF16 if dtype == W.BF16 else pa.PA_F32)
    pa.pa_copy_pages(kt, vt, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), desc=desc)
    torch.cuda.synchronize()
    k2, v2 = ORACLE.copy_pages(kp, vp, src, dst)
    assert np.array_equal(raw(kt).view(np.uint8), k2.view(np.uint8))
    assert np.array_equal(raw(vt).view(np.uint8), v2.view(np.uint8))


def test_shared_prefix_pages_with_copy_on_write():
    """Request A prefills a 70-token prompt; B and C fork A's first 70 keys
    (five pages: four full and one partial) and then decode and append their
    own tokens.  The first append into the shared partial page takes a
    private copy (pool.cow + pa_copy_pages), so A's cache never changes under
    it.  Every step's attention for all three requests matches the oracle on
    the oracle's own copy of the pools, and A's prefix pages stay shared."""
    rng = np.random.default_rng(8)
    Hq, Hkv, d, P = 8, 2, 128, 16
    NP, MP = 32, 12
    pool = pa.PagePool(NP)
    k_pool = torch.zeros(NP, Hkv, P, d, dtype=torch.bfloat16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    kp_host = np.zeros((NP, Hkv, P, d), np.uint16)
    vp_host = np.zeros_like(kp_host)
    table = np.full((3, MP), -1, np.int32)
    scale = 1.0 / np.sqrt(d)
    desc_copy = pa.pa_desc(1, Hkv, Hkv, d, P, NP, MP, 1, P, 1, pa.PA_BF16)

    def step(active, lens, n, label):
        nonlocal kp_host, vp_host
        rows = int(sum(n))
        offs = np.array(lens, np.int64)
        new = offs + np.array(n, np.int64)
        kn = W.f32_to_bf16_bits(rng.standard_normal((rows, Hkv, d)).astype(np.float32))
        vn = W.f32_to_bf16_bits(rng.standard_normal((rows, Hkv, d)).astype(np.float32))
        q = W.f32_to_bf16_bits(rng.standard_normal((rows, Hq, d)).astype(np.float32))
        t = table[active].copy()
        sl = torch.from_numpy(new.astype(np.int32)).cuda()
        qo = torch.from_numpy(offs.astype(np.int32)).cuda()
        pt = torch.from_numpy(t).cuda()
        pa.pa_append_kv(to_torch(kn, W.BF16), to_torch(vn, W.BF16), k_pool, v_pool, pt, sl, qo,
                        max_seq_len=int(new.max()), max_q_len=int(max(n)))
        kp_host, vp_host = ORACLE.append_kv(kp_host, vp_host, t, new, offs, kn, vn)
        qt = to_torch(q, W.BF16)
        if max(n) > 1:
            out, lse = pa.pa_prefill_chunk(qt, k_pool, v_pool, pt, sl, qo, scale,
                                           max_seq_len=int(new.max()), max_q_len=int(max(n)))
        else:
            out, lse = pa.pa_decode(qt, k_pool, v_pool, pt, sl, qo, scale, max_seq_len=int(new.max()))
        torch.cuda.synchronize()
        assert np.array_equal(raw(k_pool).view(np.uint8), kp_host.view(np.uint8))
        assert np.array_equal(raw(v_pool).view(np.uint8), vp_host.view(np.uint8))
        b = W.PagedBatch(name=label, seed=0, q=q, k_pool=kp_host, v_pool=vp_host, page_table=t,
                         seq_lens=new.astype(np.int32), q_offsets=offs.astype(np.int32), num_q_heads=Hq,
                         num_kv_heads=Hkv, head_dim=d, page_size=P, scale=scale, dtype=W.BF16)
        ro, rl = oracle_run(b)
        compare(b, out, lse, ro, rl, label=label)
        return [int(x) for x in new]

    # A prefills its prompt
    pool.reserve(table[0], 0, 70, P)
    (len_a,) = step([0], [0], [70], "A prompt")
    prefix_pages = table[0, :5].copy()
    a_prefix_k = raw(k_pool)[prefix_pages].copy()
    # B and C start from A's prefix
    pool.fork(table[0], table[1], 70, P)
    pool.fork(table[0], table[2], 70, P)
    assert [pool.refcount(i) for i in prefix_pages] == [3] * 5
    lens = [len_a, 70, 70]
    for it in range(20):
        for r in (1, 2, 0):
            lp = lens[r] // P                      # the page this request writes next
            if lp < MP and table[r, lp] >= 0:
                old, new = pool.cow(table[r], lp)
                if old != new:                     # shared: copy before writing
                    pa.pa_copy_pages(k_pool, v_pool, torch.tensor([old], dtype=torch.int32, device="cuda"),
                                     torch.tensor([new], dtype=torch.int32, device="cuda"), desc=desc_copy)
                    kp_host, vp_host = ORACLE.copy_pages(kp_host, vp_host, [old], [new])
            pool.reserve(table[r], lens[r], lens[r] + 1, P)
        lens = step([0, 1, 2], lens, [1, 1, 1], f"decode {it}")
    # the full prefix pages are still shared by all three; the partial one was copied
    assert [pool.refcount(i) for i in prefix_pages[:4]] == [3] * 4
    assert table[1, 4] != prefix_pages[4] and table[2, 4] != prefix_pages[4]
    # A's own appends went into its partial page 4 and beyond, never into B's or C's copies
    assert np.array_equal(raw(k_pool)[prefix_pages[:4]], a_prefix_k[:4])
