"""GPU parity of the chunked-prefill path (bf16 MFMA) against the CPU oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import paged_kv_cache_02_amd as pa
import workloads as W
from helpers import LSE_TOL, OUT_TOL_BF16, STRESS_REL, compare, device_batch, oracle_run, out_to_f64

pytestmark = pytest.mark.gpu


def run_prefill(b, dev=None, q_starts=None):
    dev = dev or device_batch(b)
    torch.cuda.synchronize()
    out, lse = pa.pa_prefill_chunk(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                   dev["seq_lens"], dev["q_offsets"], b.scale, q_starts=q_starts,
                                   max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    return out, lse


def chunk_batch(seed, seq_lens, q_offsets, Hq, Hkv, d, **kw):
    return W.make_batch(f"chunks{seed}", seed, np.array(seq_lens, np.int32),
                        np.array(q_offsets, np.int32), Hq, Hkv, d, 16, W.BF16, **kw)


def test_mixed_step_prefill_chunks_full():
    full = W.make_config("mixed_step")
    b = full.subset(*full.notes["prefill_requests"], name="mixed prefill chunks")
    print("case mixed_step prefill chunks 4x512 at offsets 0/512/1536/3072", flush=True)
    out, lse = run_prefill(b)
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label="mixed-step prefill")


@pytest.mark.parametrize("seed", [11, 12, 13, 14, 15])
def test_mixed_step_prefill_chunks_other_seeds(seed):
    # the mixed step's chunk shapes (512 tokens at offsets 0/512/1536/3072)
    # drawn from five more seeds, each compared on every row at the plain bar
    full = W.make_config("mixed_step", seed=seed)
    b = full.subset(*full.notes["prefill_requests"], name=f"mixed prefill chunks seed {seed}")
    print(f"case mixed_step prefill chunks seed {seed}", flush=True)
    out, lse = run_prefill(b)
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label=f"mixed-step prefill seed {seed}")


def few_dominant_keys_batch(seed):
    """A 512-token chunk at offset 0 whose rows are dominated by a few keys:
    scores x4, the V rows of the first 32 keys pushed to |v| in [3, 3.875],
    every V clipped to |v| <= 3.875.  Early rows then average a handful of
    large values, which is where the precision of the weights in the P V
    product shows.  |out| stays below 4, the range where a bf16 output step
    (2^-7 at most) leaves room under the 1e-2 bar."""
    b = chunk_batch(seed, [512], [0], 32, 8, 128)
    b.q = W.f32_to_bf16_bits(b.q_f32() * 4.0)
    vp = b.v_pool_f32().copy()
    for pg in b.page_table[0, :2]:
        x = vp[pg]
        vp[pg] = np.sign(x) * (3.0 + 0.875 * np.abs(np.tanh(x)))
    b.v_pool = W.f32_to_bf16_bits(np.clip(vp, -3.875, 3.875))
    return b


@pytest.mark.parametrize("seed", [100, 101, 102])
def test_rows_dominated_by_few_large_values(seed):
    b = few_dominant_keys_batch(seed)
    print(f"case few dominant keys seed {seed}", flush=True)
    out, lse = run_prefill(b)
    ro, rl = oracle_run(b)
    st = compare(b, out, lse, ro, rl, label=f"prefill few dominant keys seed {seed}")
    assert st["max_abs_oracle_out"] < 4.0


def test_values_near_the_fp16_range():
    # the P V product runs on fp16 operands: V of magnitude up to 6e4 (below
    # fp16's 65504) must come through finite and as precise, relative to the
    # size of V, as unit-scale V is: the error is held to 2^-8 of max |v|
    # (an output in [2^15, 2^16) rounds to a multiple of 256, up to 2^-8.9 of
    # 6e4, and the rest is a small share of that).  An output near zero is
    # a cancellation of large values, so its error is measured against the
    # scale of V, not against itself.
    b = chunk_batch(59, [300, 130], [0, 64], 32, 8, 128)
    vp = b.v_pool_f32().copy()
    vp = np.sign(vp) * np.minimum(np.abs(vp) * 2.0e4, 6.0e4)
    b.v_pool = W.f32_to_bf16_bits(vp)
    vmax = float(np.nanmax(np.abs(b.v_pool_f32())))
    out, lse = run_prefill(b)
    ro, rl = oracle_run(b)
    o = out_to_f64(out)
    assert np.all(np.isfinite(o))
    err = np.abs(o - ro).max() / vmax
    print(f"[fp16 range] max |d out| / max |v| = {err:.3e}, max |v| = {vmax:.0f}", flush=True)
    assert 50000.0 < vmax < 65504.0
    assert err <= 2.0 ** -8
    assert np.max(np.abs(lse.cpu().numpy() - rl)) <= LSE_TOL


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 128), (16, 8, 128), (8, 8, 128), (64, 8, 128),
                                      (32, 8, 64), (4, 4, 64), (16, 1, 64),
                                      (24, 8, 128), (48, 8, 128), (28, 4, 128), (48, 4, 64),
                                      (24, 1, 128)])
def test_ragged_chunks(Hq, Hkv, d):
    # chunk lengths not multiples of the 128-row tile, offsets not page-aligned,
    # a one-token chunk, a chunk starting at 0 and a chunk spanning many pages
    L = [45, 300, 1, 77, 1000, 130]
    o = [0, 170, 0, 76, 357, 2]
    b = chunk_batch(200 + Hq + d, L, o, Hq, Hkv, d)
    print(f"case ragged chunks Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    out, lse = run_prefill(b)
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label=f"prefill G={Hq // Hkv} d={d}")


def test_q_starts_given_or_derived_is_bit_identical():
    b = chunk_batch(51, [100, 333, 64], [10, 200, 0], 32, 8, 128)
    dev = device_batch(b)
    out1, lse1 = run_prefill(b, dev)
    qs = torch.from_numpy(b.q_row_starts.astype(np.int32)).cuda()
    out2, lse2 = run_prefill(b, dev, q_starts=qs)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_page_permutation_gives_bit_identical_output():
    b = chunk_batch(52, [700, 250], [300, 0], 32, 8, 128, pool_factor=2.0)
    out1, lse1 = run_prefill(b)
    rng = np.random.default_rng(9)
    perm = rng.permutation(b.num_pages)
    kp = np.empty_like(b.k_pool)
    vp = np.empty_like(b.v_pool)
    kp[perm] = b.k_pool
    vp[perm] = b.v_pool
    b.k_pool, b.v_pool = kp, vp
    b.page_table = np.where(b.page_table >= 0, perm[np.maximum(b.page_table, 0)], -1).astype(np.int32)
    out2, lse2 = run_prefill(b)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_last_row_matches_decode_of_that_position():
    b = chunk_batch(53, [900], [500], 32, 8, 128)
    out, lse = run_prefill(b)
    dec = chunk_batch(53, [900], [899], 32, 8, 128)
    # same pool, same page table; the decode query is the chunk's last row
    dec.k_pool, dec.v_pool, dec.page_table = b.k_pool, b.v_pool, b.page_table
    dec.q = b.q[-1:].copy()
    dd = device_batch(dec)
    out_d, lse_d = pa.pa_decode(dd["q"], dd["k_pool"], dd["v_pool"], dd["page_table"],
                                dd["seq_lens"], dd["q_offsets"], dec.scale, max_seq_len=900)
    torch.cuda.synchronize()
    assert np.max(np.abs(out_to_f64(out[-1:]) - out_to_f64(out_d))) <= 2 * OUT_TOL_BF16
    assert np.max(np.abs(lse[-1:].cpu().numpy() - lse_d.cpu().numpy())) <= LSE_TOL


def test_large_scores_stay_finite():
    b = chunk_batch(54, [400, 90], [100, 0], 32, 8, 128)
    b.q = W.f32_to_bf16_bits(b.q_f32() * 30.0)
    out, lse = run_prefill(b)
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label="prefill scores x30", rel=STRESS_REL)


def test_zero_query_gives_running_mean():
    b = chunk_batch(55, [77, 200], [0, 150], 8, 8, 128)
    b.q[:] = 0
    out, lse = run_prefill(b)
    pos = np.concatenate([np.arange(0, 77), np.arange(150, 200)]).astype(np.float64)
    assert np.max(np.abs(lse.cpu().numpy() - np.log(pos + 1)[:, None])) < LSE_TOL
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label="prefill q = 0")


def test_nan_poison_does_not_leak():
    b = chunk_batch(56, [33, 19, 250], [1, 0, 245], 32, 8, 128, pool_factor=3.0)
    assert np.isnan(b.v_pool_f32()).any() and (b.page_table == -1).any()
    out, lse = run_prefill(b)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    ro, rl = oracle_run(b)
    compare(b, out, lse, ro, rl, label="prefill poisoned pool")


def test_repeated_runs_are_bit_identical():
    b = chunk_batch(57, [600, 1200], [88, 700], 32, 8, 128)
    dev = device_batch(b)
    o1, l1 = run_prefill(b, dev)
    o2, l2 = run_prefill(b, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_long_context_short_chunk_splits_across_workgroups():
    # one short chunk deep into a long context: few query tiles, so the guard
    # also splits each tile's key range across workgroups (partials + merge
    # pass); the unsplit route must agree with the oracle too
    b = chunk_batch(58, [4100, 2500], [4036, 2480], 32, 8, 128)
    dev = device_batch(b)
    desc = pa.make_desc(dev["q"], dev["k_pool"], dev["page_table"], dev["seq_lens"], b.max_seq_len,
                        b.max_q_len)
    plan = pa.pa_plan(desc)
    print(f"case short chunk deep in context plan={plan}", flush=True)
    assert plan["num_splits"] > 1 and plan["workspace_bytes"] > 0
    ro, rl = oracle_run(b)
    out, lse = run_prefill(b, dev)
    compare(b, out, lse, ro, rl, label="prefill split across workgroups")
    out2, lse2 = pa.pa_prefill_chunk(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                     dev["seq_lens"], dev["q_offsets"], b.scale, split=False,
                                     max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
    torch.cuda.synchronize()
    compare(b, out2, lse2, ro, rl, label="prefill unsplit")


def test_groups_starting_past_the_read_ahead_tiles():
    # a chunk at the end of a 9000-key context: the second wave group starts
    # at KV tile 71, past the 64 tiles whose page ids the prologue reads
    # ahead, so its first page id comes straight from the table; the split
    # route's later splits start past tile 64 as well
    b = chunk_batch(59, [9000, 1000], [8800, 900], 32, 8, 128, pool_factor=1.2)
    dev = device_batch(b)
    print("case prefill groups past the read-ahead tiles", flush=True)
    ro, rl = oracle_run(b)
    for split in (False, True):
        out, lse = pa.pa_prefill_chunk(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                       dev["seq_lens"], dev["q_offsets"], b.scale, split=split,
                                       max_seq_len=b.max_seq_len, max_q_len=b.max_q_len)
        torch.cuda.synchronize()
        compare(b, out, lse, ro, rl, label=f"prefill past the read-ahead tiles split={split}")


def test_bound_call_matches_the_wrapper():
    b = chunk_batch(77, [600, 300, 129], [88, 0, 1], 32, 8, 128)
    dev = device_batch(b)
    ref, ref_lse = run_prefill(b, dev)
    desc = pa.make_desc(dev["q"], dev["k_pool"], dev["page_table"], dev["seq_lens"], b.max_seq_len,
                        b.max_q_len)
    need = pa.pa_plan(desc)["workspace_bytes"]
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    out, lse = torch.empty_like(ref), torch.empty_like(ref_lse)
    call = pa.bind_prefill_chunk(dev["q"], dev["k_pool"], dev["v_pool"], dev["page_table"],
                                 dev["seq_lens"], dev["q_offsets"], b.scale, q_starts=None,
                                 out=out, lse=lse, workspace=ws, desc=desc)
    for _ in range(3):
        out.zero_()
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
