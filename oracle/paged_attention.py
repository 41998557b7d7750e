"""CPU oracle for attention read out of a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's GPU path
never calls it, and it shares no code with the GPU path.

What is computed.  The pages describe a KV cache kept as fixed-size pages in
one shared pool, with a per-request page table mapping logical pages to
physical pages, and an attention that reads the pages through that table and
folds the page addressing together with online softmax (tiny-llm source
reading, yangyang233333.github.io, section "Paged KV Cache" of week 3; the
same pair of items in the week-3 list of "Build a vLLM from Scratch",
blog.mushroom.cv).  The attention itself is never written out on the pages, so
this oracle takes the textbook definition of scaled dot-product attention with
grouped-query heads and a causal mask (the week-1 items of the tiny-llm source
reading: GQA, causal mask), computed the plain way:

  1. gather: key j of request r lives at page page_table[r][j // P], slot j % P
  2. visible keys of the query row at absolute position p: 0 <= j <= p
  3. pass 1: s_j = scale * (q . k_j) in float64, m = max_j s_j
  4. pass 2: w_j = exp(s_j - m), l = sum_j w_j, out = sum_j w_j v_j / l,
             lse = m + ln l

Online softmax is a reordering of steps 3-4 that the GPU path uses; the oracle
deliberately does not use it.  The split-K partials and their logsumexp merge
(Flash-Decoding split-K for long decode contexts, mini-vllm-tutorial advanced
series design, item adv04) are defined the same way on page ranges, merged by
the log-sum-exp rule written out in `merge`.

Readings taken where the pages are silent:
  * query head h uses KV head h // G with G = Hq / Hkv (consecutive grouping);
  * seq_lens[r] counts the keys already appended for this step, so a request
    has n_r = seq_lens[r] - q_offsets[r] query rows at absolute positions
    q_offsets[r] .. seq_lens[r]-1 (a decode row is the case n_r = 1);
  * lse is the natural log of the sum of exp of the scaled scores;
  * split s of request r covers the page range [a_s, b_s) chosen by the
    caller; an empty range has lse = -inf and a zero partial output.

Parity pins: every function here is pinned by tests that do not reuse this
module's arithmetic (hand-computed page addresses, torch's scaled-dot-product
attention on float64 tensors, a pure-Python scalar triple loop, closed forms
for a single key and for equal scores, page-permutation invariance, and
merge(split) = unsplit).  No function is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# page-table translation
# ----------------------------------------------------------------------------
def gather(k_pool: np.ndarray, v_pool: np.ndarray, page_table_row: np.ndarray,
           seq_len: int) -> Tuple[np.ndarray, np.ndarray]:
    """Copy the first seq_len keys of one request out of the pool.

    k_pool, v_pool: [NP, Hkv, P, d]; page_table_row: [MP] physical page ids.
    Returns K, V of shape [seq_len, Hkv, d] holding the stored values exactly
    (same dtype as the pool).  Logical key j is slot j % P of physical page
    page_table_row[j // P] (the page-table mapping of the paged KV cache).
    """
    P = k_pool.shape[2]
    Hkv, d = k_pool.shape[1], k_pool.shape[3]
    K = np.empty((seq_len, Hkv, d), dtype=k_pool.dtype)
    V = np.empty((seq_len, Hkv, d), dtype=v_pool.dtype)
    for j in range(seq_len):
        page = int(page_table_row[j // P])
        slot = j % P
        K[j] = k_pool[page, :, slot, :]
        V[j] = v_pool[page, :, slot, :]
    return K, V


# ----------------------------------------------------------------------------
# attention of a set of query rows against one request's contiguous keys
# ----------------------------------------------------------------------------
def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, positions: Sequence[int],
           scale: float, key_range: Tuple[int, int] = None):
    """Two-pass softmax attention in float64.

    q_rows: [n, Hq, d]; K, V: [L, Hkv, d]; positions[i] = absolute position of
    row i (it sees keys j <= positions[i]).  key_range optionally restricts the
    keys to [a, b) (a split partition).  Returns out [n, Hq, d] and lse [n, Hq]
    in float64; a row with no visible key in the range gets out = 0 and
    lse = -inf.
    """
    q64 = np.asarray(q_rows, dtype=np.float64)
    K64 = np.asarray(K, dtype=np.float64)
    V64 = np.asarray(V, dtype=np.float64)
    n, Hq, d = q64.shape
    L, Hkv, _ = K64.shape
    G = Hq // Hkv
    a, b = (0, L) if key_range is None else key_range
    out = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.full((n, Hq), -np.inf, dtype=np.float64)
    for i in range(n):
        hi = min(b, int(positions[i]) + 1)          # keys a .. hi-1 are visible
        if hi <= a:
            continue
        for h in range(Hq):
            g = h // G
            k = K64[a:hi, g, :]                      # [m, d]
            v = V64[a:hi, g, :]
            s = scale * (k @ q64[i, h])              # pass 1: scores
            m = s.max()
            w = np.exp(s - m)                        # pass 2: weights
            l = w.sum()
            out[i, h] = (w @ v) / l
            lse[i, h] = m + math.log(l)
    return out, lse


def query_positions(seq_len: int, q_offset: int) -> np.ndarray:
    """Absolute positions of a request's query rows: q_offset .. seq_len-1."""
    return np.arange(q_offset, seq_len, dtype=np.int64)


def q_row_starts(seq_lens: np.ndarray, q_offsets: np.ndarray) -> np.ndarray:
    """[B+1]: first packed query row of each request (rows ordered by request)."""
    n = np.asarray(seq_lens, np.int64) - np.asarray(q_offsets, np.int64)
    starts = np.zeros(n.size + 1, dtype=np.int64)
    for r in range(n.size):
        starts[r + 1] = starts[r] + n[r]
    return starts


def paged_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                    page_table: np.ndarray, seq_lens: np.ndarray, q_offsets: np.ndarray,
                    scale: float, requests: Sequence[int] = None):
    """Attention of every packed query row against its request's paged keys.

    q: [total_q, Hq, d] (float values); pools [NP, Hkv, P, d]; page_table
    int32 [B, MP]; seq_lens, q_offsets int32 [B].  Returns float64 out
    [total_q, Hq, d] and lse [total_q, Hq].  `requests` restricts the work to
    some requests (their rows are filled, the others stay NaN), which keeps
    the large workloads' memory bounded to one request at a time.
    """
    starts = q_row_starts(seq_lens, q_offsets)
    total_q, Hq, d = q.shape
    out = np.full((total_q, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((total_q, Hq), np.nan, dtype=np.float64)
    reqs = range(len(seq_lens)) if requests is None else requests
    for r in reqs:
        L, o = int(seq_lens[r]), int(q_offsets[r])
        K, V = gather(k_pool, v_pool, page_table[r], L)
        rows = slice(int(starts[r]), int(starts[r + 1]))
        out[rows], lse[rows] = attend(q[rows], K, V, query_positions(L, o), scale)
    return out, lse


# ----------------------------------------------------------------------------
# split-K partitions and their merge
# ----------------------------------------------------------------------------
def split_page_ranges(num_pages: int, pages_per_split: int, num_splits: int) -> List[Tuple[int, int]]:
    """Page ranges of splits 0..num_splits-1: split s covers pages
    [s * pps, min((s+1) * pps, num_pages)), empty once s * pps >= num_pages."""
    ranges = []
    for s in range(num_splits):
        a = min(s * pages_per_split, num_pages)
        b = min((s + 1) * pages_per_split, num_pages)
        ranges.append((a, b))
    return ranges


def pages_per_split_even(num_pages: int, num_splits: int) -> int:
    """Equal page counts per split: ceil(num_pages / num_splits)."""
    return -(-num_pages // num_splits)


def split_partials(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, positions, scale: float,
                   page_ranges: Sequence[Tuple[int, int]], page_size: int):
    """Per-split normalized partial outputs O_s [S, n, Hq, d] and lse_s [S, n, Hq]:
    attention restricted to the keys of the split's pages."""
    parts_o, parts_l = [], []
    for (a, b) in page_ranges:
        o, l = attend(q_rows, K, V, positions, scale,
                      key_range=(a * page_size, min(b * page_size, K.shape[0])))
        parts_o.append(o)
        parts_l.append(l)
    return np.stack(parts_o), np.stack(parts_l)


def merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Log-sum-exp merge of split partials along axis 0.

    LSE = M + ln sum_s exp(lse_s - M) with M = max over the finite lse_s;
    out = sum_s exp(lse_s - LSE) * O_s.  Splits with lse_s = -inf carry zero
    weight.  Works elementwise over the remaining axes.
    """
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    M = np.max(l, axis=0)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(l), np.exp(l - Msafe[None]), 0.0)
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        LSE = np.where(finite, Msafe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = np.where(finite[None], w / np.where(finite, tot, 1.0)[None], 0.0)
    out = (wn[..., None] * o).sum(axis=0)
    return out, LSE
