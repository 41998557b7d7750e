"""Pins for the CPU oracle.

Each pin checks the oracle against something other than itself: the
hand-written page-table fixture, torch's scaled-dot-product attention on
float64 CPU tensors (a library routine), a pure-Python scalar triple loop,
closed forms (single key, equal scores), page-permutation invariance and the
identity merge(split) = unsplit.  Every pin takes the oracle module as an
argument so that `test_mutants_are_caught` can run the same pins against
copies of the oracle with a planted mistake and check that one of them fails.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle as ORACLE
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers that do not use the oracle
# ----------------------------------------------------------------------------
def contiguous_kv_identity(batch, r):
    """K, V of request r for a batch built with pool='identity': the request's
    pages are consecutive in the pool, so its keys are a reshape of a slice."""
    P = batch.page_size
    npg = (int(batch.seq_lens[r]) + P - 1) // P
    first = int(batch.page_table[r, 0])
    L = int(batch.seq_lens[r])
    k = batch.k_pool_f32()[first:first + npg].transpose(0, 2, 1, 3).reshape(npg * P, batch.num_kv_heads, -1)[:L]
    v = batch.v_pool_f32()[first:first + npg].transpose(0, 2, 1, 3).reshape(npg * P, batch.num_kv_heads, -1)[:L]
    return k.astype(np.float64), v.astype(np.float64)


def sdpa_request(batch, r, q_rows, K, V, causal_offset):
    """torch SDPA in float64 for one request: q_rows [n,Hq,d], K,V [L,Hkv,d]."""
    n = q_rows.shape[0]
    L = K.shape[0]
    q = torch.from_numpy(np.ascontiguousarray(q_rows.transpose(1, 0, 2)))[None]
    k = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    v = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    i = torch.arange(n)[:, None]
    j = torch.arange(L)[None, :]
    mask = j <= (causal_offset + i)
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, scale=batch.scale, enable_gqa=True)
    # lse via torch's own logsumexp on explicitly masked scores
    G = batch.num_q_heads // batch.num_kv_heads
    kr = k.repeat_interleave(G, dim=1)
    s = (q @ kr.transpose(-1, -2)) * batch.scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return out[0].numpy().transpose(1, 0, 2), lse[0].numpy().T


def small_batch(seed=7, seq_lens=(5, 23, 40), q_offsets=None, Hq=4, Hkv=2, d=8, P=4, pool="permuted",
                dtype=W.F32, num_pages=None):
    seq_lens = np.array(seq_lens, np.int32)
    q_offsets = seq_lens - 1 if q_offsets is None else np.array(q_offsets, np.int32)
    return W.make_batch("small", seed, seq_lens, q_offsets, Hq, Hkv, d, P, dtype, pool=pool,
                        num_pages=num_pages)


def run_oracle(O, b, **kw):
    return O.paged_attention(b.q_f32(), b.k_pool_f32(), b.v_pool_f32(), b.page_table, b.seq_lens,
                             b.q_offsets, b.scale, **kw)


# ----------------------------------------------------------------------------
# pins (each takes the oracle module)
# ----------------------------------------------------------------------------
def pin_page_table_fixture(O):
    rows = []
    with open(os.path.join(GOLDEN, "page_table_example.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                req, j, page, slot = line.split()
                rows.append((req, int(j), int(page), int(slot)))
    P, Hkv, d, NP = 4, 2, 3, 12
    pool = np.zeros((NP, Hkv, P, d))
    for p in range(NP):
        for g in range(Hkv):
            for s in range(P):
                for c in range(d):
                    pool[p, g, s, c] = 1000 * p + 100 * g + 10 * s + c
    tables = {"A": np.array([7, 2, 11, -1], np.int32), "B": np.array([4, 9, -1, -1], np.int32)}
    lens = {"A": 10, "B": 7}
    for req in ("A", "B"):
        K, V = O.gather(pool, -pool, tables[req], lens[req])
        assert K.shape == (lens[req], Hkv, d)
        expect = [(j, page, slot) for (rq, j, page, slot) in rows if rq == req]
        assert len(expect) == lens[req]
        for (j, page, slot) in expect:
            for g in range(Hkv):
                for c in range(d):
                    want = 1000 * page + 100 * g + 10 * slot + c
                    assert K[j, g, c] == want and V[j, g, c] == -want, (req, j, g, c)


def pin_identity_table_matches_sdpa(O):
    b = small_batch(seed=11, seq_lens=(9, 33, 64, 17), q_offsets=(0, 20, 63, 3), pool="identity")
    out, lse = run_oracle(O, b)
    starts = b.q_row_starts
    for r in range(b.num_seqs):
        K, V = contiguous_kv_identity(b, r)
        rows = slice(starts[r], starts[r + 1])
        ro, rl = sdpa_request(b, r, b.q_f32()[rows].astype(np.float64), K, V, int(b.q_offsets[r]))
        assert np.max(np.abs(out[rows] - ro)) < 1e-12
        assert np.max(np.abs(lse[rows] - rl)) < 1e-12


def pin_bruteforce_tiny(O):
    b = W.make_config("tiny_decode")
    out, lse = run_oracle(O, b)
    q, kp, vp = b.q_f32(), b.k_pool_f32(), b.v_pool_f32()
    P, G = b.page_size, b.num_q_heads // b.num_kv_heads
    for r in range(b.num_seqs):
        L = int(b.seq_lens[r])
        for h in range(b.num_q_heads):
            g = h // G
            scores = []
            for j in range(L):
                page, slot = int(b.page_table[r, j // P]), j % P
                acc = 0.0
                for c in range(b.head_dim):
                    acc += float(q[r, h, c]) * float(kp[page, g, slot, c])
                scores.append(acc * b.scale)
            m = max(scores)
            ws = [math.exp(s - m) for s in scores]
            l = sum(ws)
            assert abs(lse[r, h] - (m + math.log(l))) < 1e-12
            for c in range(b.head_dim):
                num = 0.0
                for j in range(L):
                    page, slot = int(b.page_table[r, j // P]), j % P
                    num += ws[j] * float(vp[page, g, slot, c])
                assert abs(out[r, h, c] - num / l) < 1e-12


def pin_page_permutation_invariance(O):
    b = small_batch(seed=3, seq_lens=(31, 7, 50), q_offsets=(20, 6, 0), num_pages=40)
    out, lse = run_oracle(O, b)
    rng = np.random.default_rng(99)
    perm = rng.permutation(b.num_pages)           # physical page p moves to perm[p]
    kp = np.empty_like(b.k_pool)
    vp = np.empty_like(b.v_pool)
    kp[perm] = b.k_pool
    vp[perm] = b.v_pool
    table = np.where(b.page_table >= 0, perm[np.maximum(b.page_table, 0)], -1).astype(np.int32)
    out2, lse2 = O.paged_attention(b.q_f32(), W.as_f32(kp, b.dtype), W.as_f32(vp, b.dtype), table,
                                   b.seq_lens, b.q_offsets, b.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def pin_single_key(O):
    b = small_batch(seed=5, seq_lens=(1, 1), q_offsets=(0, 0), Hq=6, Hkv=3, d=16)
    out, lse = run_oracle(O, b)
    q, kp, vp = b.q_f32(), b.k_pool_f32(), b.v_pool_f32()
    G = b.num_q_heads // b.num_kv_heads
    for r in range(b.num_seqs):
        page = int(b.page_table[r, 0])
        for h in range(b.num_q_heads):
            g = h // G
            assert np.array_equal(out[r, h], vp[page, g, 0].astype(np.float64))
            dot = math.fsum(float(a) * float(c) for a, c in zip(q[r, h], kp[page, g, 0]))
            assert abs(lse[r, h] - b.scale * dot) < 1e-12


def pin_equal_scores(O):
    b = small_batch(seed=6, seq_lens=(13, 40), q_offsets=(5, 39), Hq=4, Hkv=1, d=8)
    q0 = np.zeros_like(b.q_f32())
    out, lse = O.paged_attention(q0, b.k_pool_f32(), b.v_pool_f32(), b.page_table, b.seq_lens,
                                 b.q_offsets, b.scale)
    vp = b.v_pool_f32()
    starts = b.q_row_starts
    P = b.page_size
    for r in range(b.num_seqs):
        o = int(b.q_offsets[r])
        for i in range(int(b.seq_lens[r]) - o):
            n = o + i + 1
            vals = [vp[int(b.page_table[r, j // P]), 0, j % P].astype(np.float64) for j in range(n)]
            mean = np.sum(vals, axis=0) / n
            row = starts[r] + i
            assert np.max(np.abs(out[row] - mean[None])) < 1e-12
            assert np.max(np.abs(lse[row] - math.log(n))) < 1e-12


def pin_gqa_consecutive_grouping(O):
    # Each q head h must equal plain multi-head attention against KV head h // G:
    # expand the pool's KV heads by repetition so that G becomes 1 and compare.
    b = small_batch(seed=8, seq_lens=(19, 44), q_offsets=(18, 10), Hq=6, Hkv=2, d=8)
    out, lse = run_oracle(O, b)
    G = 3
    kp = np.repeat(b.k_pool_f32(), G, axis=1)
    vp = np.repeat(b.v_pool_f32(), G, axis=1)
    out2, lse2 = O.paged_attention(b.q_f32(), kp, vp, b.page_table, b.seq_lens, b.q_offsets, b.scale)
    assert np.max(np.abs(out - out2)) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-13


def pin_prefill_row_equals_decode(O):
    b = small_batch(seed=9, seq_lens=(40,), q_offsets=(25,), Hq=4, Hkv=2, d=8)
    out, lse = run_oracle(O, b)
    for i in range(15):
        p = 25 + i
        L = np.array([p + 1], np.int32)
        od, ld = O.paged_attention(b.q_f32()[i:i + 1], b.k_pool_f32(), b.v_pool_f32(), b.page_table,
                                   L, L - 1, b.scale)
        assert np.max(np.abs(od[0] - out[i])) < 1e-13 and np.max(np.abs(ld[0] - lse[i])) < 1e-13


def pin_prefill_from_zero_is_causal_sdpa(O):
    b = small_batch(seed=10, seq_lens=(37,), q_offsets=(0,), Hq=4, Hkv=2, d=8, pool="identity")
    out, lse = run_oracle(O, b)
    K, V = contiguous_kv_identity(b, 0)
    q = torch.from_numpy(b.q_f32().astype(np.float64).transpose(1, 0, 2).copy())[None]
    k = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    v = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=b.scale,
                                                           enable_gqa=True)
    assert np.max(np.abs(out - ref[0].numpy().transpose(1, 0, 2))) < 1e-12


def pin_split_merge_identity(O):
    b = small_batch(seed=12, seq_lens=(45, 64, 3), q_offsets=(44, 40, 0), Hq=4, Hkv=2, d=8)
    out, lse = run_oracle(O, b)
    starts = b.q_row_starts
    P = b.page_size
    for r in range(b.num_seqs):
        L = int(b.seq_lens[r])
        npg = (L + P - 1) // P
        K, V = O.gather(b.k_pool_f32(), b.v_pool_f32(), b.page_table[r], L)
        rows = slice(starts[r], starts[r + 1])
        pos = O.query_positions(L, int(b.q_offsets[r]))
        for S in (1, 2, 3, 16, npg + 5):
            pps = O.pages_per_split_even(npg, S)
            ranges = O.split_page_ranges(npg, pps, S)
            # the ranges tile [0, npg) in order
            assert ranges[0][0] == 0 and ranges[-1][1] == npg
            assert all(ranges[i][1] == ranges[i + 1][0] for i in range(S - 1))
            po, pl = O.split_partials(b.q_f32()[rows], K, V, pos, b.scale, ranges, P)
            mo, ml = O.merge(po, pl)
            assert np.max(np.abs(mo - out[rows])) < 1e-12
            assert np.max(np.abs(ml - lse[rows])) < 1e-12
            if S == 1:
                assert np.max(np.abs(po[0] - out[rows])) < 1e-15


def pin_large_scores_stay_finite(O):
    b = small_batch(seed=13, seq_lens=(30, 61), q_offsets=(29, 10), Hq=4, Hkv=2, d=8, pool="identity")
    q30 = b.q_f32().astype(np.float64) * 30.0
    out, lse = O.paged_attention(q30, b.k_pool_f32(), b.v_pool_f32(), b.page_table, b.seq_lens,
                                 b.q_offsets, b.scale)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    starts = b.q_row_starts
    for r in range(b.num_seqs):
        K, V = contiguous_kv_identity(b, r)
        rows = slice(starts[r], starts[r + 1])
        ro, rl = sdpa_request(b, r, q30[rows], K, V, int(b.q_offsets[r]))
        assert np.max(np.abs(out[rows] - ro)) < 1e-10
        assert np.max(np.abs(lse[rows] - rl)) < 1e-10


def pin_q_row_starts(O):
    st = O.q_row_starts(np.array([5, 9, 1, 4]), np.array([0, 8, 0, 1]))
    assert list(st) == [0, 5, 6, 7, 10]


def pin_merge_closed_form(O):
    # two partitions with lse 0 and ln 3: weights 1/4 and 3/4, LSE = ln 4;
    # an empty partition (-inf) carries no weight
    o = np.array([[[1.0, 2.0]], [[5.0, -2.0]], [[123.0, 7.0]]])
    l = np.array([[0.0], [math.log(3.0)], [-np.inf]])
    mo, ml = O.merge(o, l)
    assert abs(ml[0] - math.log(4.0)) < 1e-15
    assert np.max(np.abs(mo[0] - np.array([0.25 * 1 + 0.75 * 5, 0.25 * 2 - 0.75 * 2]))) < 1e-15


PINS = [pin_page_table_fixture, pin_identity_table_matches_sdpa, pin_bruteforce_tiny,
        pin_page_permutation_invariance, pin_single_key, pin_equal_scores,
        pin_gqa_consecutive_grouping, pin_prefill_row_equals_decode,
        pin_prefill_from_zero_is_causal_sdpa, pin_split_merge_identity,
        pin_large_scores_stay_finite, pin_q_row_starts, pin_merge_closed_form]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(ORACLE)


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------
MUTANTS = {
    "gqa_mod_mapping": ("g = h // G", "g = h % Hkv"),
    "slot_from_page_index": ("slot = j % P", "slot = j // P % P"),
    "page_from_slot": ("page = int(page_table_row[j // P])", "page = int(page_table_row[j % P % 2])"),
    "causal_off_by_one": ("hi = min(b, int(positions[i]) + 1)", "hi = min(b, int(positions[i]) + 2)"),
    "causal_excludes_diagonal": ("hi = min(b, int(positions[i]) + 1)", "hi = min(b, max(int(positions[i]), 1))"),
    "scale_dropped": ("s = scale * (k @ q64[i, h])", "s = (k @ q64[i, h])"),
    "lse_drops_max": ("lse[i, h] = m + math.log(l)", "lse[i, h] = math.log(l)"),
    "no_normalisation": ("out[i, h] = (w @ v) / l", "out[i, h] = (w @ v)"),
    "exp_sign": ("w = np.exp(s - m)", "w = np.exp(m - s)"),
    "k_for_v": ("v = V64[a:hi, g, :]", "v = K64[a:hi, g, :]"),
    "q_transposed_heads": ("s = scale * (k @ q64[i, h])", "s = scale * (k @ q64[i, (h + 1) % Hq])"),
    "merge_weight_sign": ("np.exp(l - Msafe[None])", "np.exp(Msafe[None] - l)"),
    "merge_lse_drops_max": ("LSE = np.where(finite, Msafe + np.log(", "LSE = np.where(finite, 0 * Msafe + np.log("),
    "split_last_range": ("b = min((s + 1) * pages_per_split, num_pages)", "b = min((s + 1) * pages_per_split, num_pages - 1)"),
    "row_starts_skip": ("starts[r + 1] = starts[r] + n[r]", "starts[r + 1] = starts[r] + n[r] + (r == 1)"),
}


def _mutant_module(src, old, new):
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name):
    src = open(os.path.join(os.path.dirname(ORACLE.__file__), "paged_attention.py")).read()
    old, new = MUTANTS[name]
    mod = _mutant_module(src, old, new)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:   # assertion or crash both count as caught
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


# ----------------------------------------------------------------------------
# the input generator
# ----------------------------------------------------------------------------
def test_bf16_encoding_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e38], np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert back[1] == 1.0
    # 1 + 1.5 * 2^-8 rounds up to 1 + 2^-7
    assert back[2] == np.float32(1.0078125)
    assert back[0] == 1.0 and back[3] == np.float32(1.0078125) and back[4] == -2.5
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t, bits)


@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_0p6b_decode", "long_splitk_decode"])
def test_workload_structure(name):
    b = W.make_config(name)
    P = b.page_size
    npg = (b.seq_lens.astype(np.int64) + P - 1) // P
    used = []
    for r in range(b.num_seqs):
        row = b.page_table[r]
        assert np.all(row[:npg[r]] >= 0) and np.all(row[:npg[r]] < b.num_pages)
        assert np.all(row[npg[r]:] == -1)
        used.extend(row[:npg[r]].tolist())
    assert len(set(used)) == len(used)          # no page shared by two requests
    assert b.total_q == int((b.seq_lens - b.q_offsets).sum())
    if name == "tiny_decode":
        assert list(b.seq_lens) == [37, 100] and b.num_pages == 16 and b.dtype == W.F32
    if name == "qwen3_0p6b_decode":
        assert b.num_seqs == 32 and b.seq_lens.min() >= 128 and b.seq_lens.max() <= 2048
        assert b.num_pages == int(math.ceil(1.25 * npg.sum()))
    if name == "long_splitk_decode":
        assert b.num_pages == 16 * 2048 and b.num_splits == 16


def test_poison_only_where_no_key_lives():
    b = small_batch(seed=21, seq_lens=(5, 18), q_offsets=(4, 17), num_pages=12)
    k = b.k_pool_f32()
    live = W.live_slot_mask(b.page_table, b.seq_lens, b.num_pages, b.page_size)
    assert np.all(np.isnan(k.transpose(0, 2, 1, 3)[~live]))
    assert not np.any(np.isnan(k.transpose(0, 2, 1, 3)[live]))
