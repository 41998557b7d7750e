"""CPU oracle for appending new K/V rows into a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's GPU path
never calls it, and it shares no code with the GPU path.

What is computed.  In a serving step, every request's new tokens (a prefill
chunk, or the one token of a decode step) have their K and V rows written
into the shared pool before attention reads them: token position p of request
r goes to slot p % P of physical page page_table[r][p // P] (tiny-llm source
reading, yangyang233333.github.io, section "Paged KV Cache": pages are taken
from a shared pool on demand and the page table maps a request's logical
sequence to them; "Build a vLLM from Scratch", blog.mushroom.cv, Week 3: the
cache grows by pages instead of reserving contiguous space).

The new rows are packed like the queries of the attention entry points: rows
ordered by request, then token; request r contributes n_r = seq_lens[r] -
q_offsets[r] rows at positions q_offsets[r] .. seq_lens[r]-1 (seq_lens counts
the keys after this step's append).  The append is a copy: bit-exact, no
arithmetic.

Parity pins (tests/test_oracle_append.py): gathering the appended positions
back through the independently pinned `gather` returns the new rows exactly;
with an identity page table the pool equals a dense [B, T, Hkv, d] cache
written by slicing; every slot that no new row maps to is left unchanged.

`copy_pages` is the device half of a copy on write for shared prefix pages
("mini-vllm-tutorial advanced-series design", Phase C, adv05: pages shared
by several requests are copied before one of them writes): page dst[i]
becomes a copy of page src[i], K and V, every KV head.  Pins: a table that
names dst gathers what the same table naming src gathered; every other page
is unchanged.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def append_kv(k_pool: np.ndarray, v_pool: np.ndarray, page_table: np.ndarray,
              seq_lens: np.ndarray, q_offsets: np.ndarray, k_new: np.ndarray,
              v_new: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools with the new rows written in.

    k_pool, v_pool: [NP, Hkv, P, d]; page_table: [B, MP]; seq_lens,
    q_offsets: [B]; k_new, v_new: [sum_r n_r, Hkv, d], rows by request then
    token.  Any dtype (values are copied, not converted).
    """
    P = k_pool.shape[2]
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    row = 0
    for r in range(len(seq_lens)):
        for pos in range(int(q_offsets[r]), int(seq_lens[r])):
            page = int(page_table[r][pos // P])
            slot = pos % P
            k_out[page, :, slot, :] = k_new[row]
            v_out[page, :, slot, :] = v_new[row]
            row += 1
    assert row == k_new.shape[0], "k_new rows must equal sum of seq_lens - q_offsets"
    return k_out, v_out


def copy_pages(k_pool: np.ndarray, v_pool: np.ndarray, src, dst) -> Tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools with page dst[i] replaced by page src[i]
    (K and V, all KV heads).  Pairs naming a page outside the pool, or the
    same page twice, are skipped."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    num_pages = k_pool.shape[0]
    for s_id, d_id in zip(src, dst):
        s_id, d_id = int(s_id), int(d_id)
        if not (0 <= s_id < num_pages and 0 <= d_id < num_pages) or s_id == d_id:
            continue
        k_out[d_id] = k_pool[s_id]
        v_out[d_id] = v_pool[s_id]
    return k_out, v_out
