"""Seeded synthetic inputs for paged attention.

This module builds the inputs that both the GPU library and the CPU oracle
consume: a shared pool of fixed-size K/V pages, per-request int32 page tables,
context lengths, query offsets and query rows.  It holds none of the attention
arithmetic -- only random draws, page assignment and bf16 storage encoding.

Layouts (shared by every consumer):
  k_pool, v_pool : [num_pages, Hkv, P, d]   (one (page, kv head) block of P*d
                                             elements is contiguous)
  page_table     : int32 [B, max_pages_per_seq], row r lists request r's
                   physical pages in logical order; entries past the request's
                   last page are -1
  seq_lens       : int32 [B]  keys held by request r (including this step's)
  q_offsets      : int32 [B]  absolute position of request r's first query row
  q              : [sum_r (L_r - o_r), Hq, d], rows ordered by request, then
                   token; heads inner

bf16 tensors are stored as numpy uint16 bit patterns (IEEE bfloat16); fp32
tensors as float32.  `as_f32` decodes either to exact float32 values.

Page-pool shapes follow the paged KV cache the tiny-llm source reading
describes (section on the paged KV cache: fixed-size pages in one shared pool,
each request holding a page table); the per-config head shapes are those of
the Qwen3 and Llama-3.2-1B families the pages name.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"

BF16_NAN_BITS = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bf16 storage encoding (round to nearest even), used only to store inputs
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(arr) if dtype == BF16 else np.asarray(arr, dtype=np.float32)


# ----------------------------------------------------------------------------
# the batch container
# ----------------------------------------------------------------------------
@dataclass
class PagedBatch:
    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    seq_lens: np.ndarray          # int32 [B]
    q_offsets: np.ndarray         # int32 [B]
    page_table: np.ndarray        # int32 [B, MP]
    k_pool: np.ndarray            # [NP, Hkv, P, d] uint16 (bf16) or float32
    v_pool: np.ndarray
    q: np.ndarray                 # [total_q, Hq, d]
    scale: float
    num_splits: Optional[int] = None
    notes: dict = field(default_factory=dict)

    # -- derived sizes -------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def q_lens(self) -> np.ndarray:
        return (self.seq_lens.astype(np.int64) - self.q_offsets.astype(np.int64)).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def q_row_starts(self) -> np.ndarray:
        """[B+1] exclusive prefix sum of the per-request query row counts."""
        out = np.zeros(self.num_seqs + 1, dtype=np.int64)
        np.cumsum(self.q_lens, out=out[1:])
        return out

    def q_f32(self) -> np.ndarray:
        return as_f32(self.q, self.dtype)

    def k_pool_f32(self) -> np.ndarray:
        return as_f32(self.k_pool, self.dtype)

    def v_pool_f32(self) -> np.ndarray:
        return as_f32(self.v_pool, self.dtype)

    def subset(self, start: int, stop: int, name: Optional[str] = None) -> "PagedBatch":
        """Requests [start, stop) as a batch that shares this batch's pool."""
        rs = self.q_row_starts
        return PagedBatch(
            name=name or f"{self.name}[{start}:{stop}]", seed=self.seed, dtype=self.dtype,
            num_q_heads=self.num_q_heads, num_kv_heads=self.num_kv_heads,
            head_dim=self.head_dim, page_size=self.page_size,
            seq_lens=self.seq_lens[start:stop], q_offsets=self.q_offsets[start:stop],
            page_table=self.page_table[start:stop], k_pool=self.k_pool, v_pool=self.v_pool,
            q=self.q[rs[start]:rs[stop]], scale=self.scale, num_splits=self.num_splits,
            notes=dict(self.notes))

    def kv_bytes(self) -> int:
        """K and V bytes of the visible keys: each key's d values, per KV head."""
        es = 2 if self.dtype == BF16 else 4
        return int(self.seq_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * es


# ----------------------------------------------------------------------------
# page assignment
# ----------------------------------------------------------------------------
def pages_for(seq_lens: np.ndarray, page_size: int) -> np.ndarray:
    return (seq_lens.astype(np.int64) + page_size - 1) // page_size


def assign_pages_permuted(rng, n_pages: np.ndarray, num_pages: int) -> np.ndarray:
    """Draw a random permutation of the pool; request r takes the next
    n_pages[r] entries of it, in request order."""
    total = int(n_pages.sum())
    assert num_pages >= total
    perm = rng.permutation(num_pages).astype(np.int32)
    mp = int(n_pages.max()) if n_pages.size else 1
    table = np.full((n_pages.size, max(mp, 1)), -1, dtype=np.int32)
    pos = 0
    for r, n in enumerate(n_pages):
        table[r, :n] = perm[pos:pos + n]
        pos += n
    return table


def assign_pages_interleaved(n_pages: np.ndarray) -> np.ndarray:
    """Fragmented pool grown round-robin: at growth step k every request that
    still needs a k-th page takes the next sequential physical page, so
    consecutive logical pages of one request are far apart in the pool."""
    mp = int(n_pages.max())
    table = np.full((n_pages.size, mp), -1, dtype=np.int32)
    nxt = 0
    for k in range(mp):
        for r in range(n_pages.size):
            if k < n_pages[r]:
                table[r, k] = nxt
                nxt += 1
    return table


# ----------------------------------------------------------------------------
# value generation
# ----------------------------------------------------------------------------
def _normal(rng, shape, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) float32 draws stored in `dtype`, generated in chunks to bound
    host memory for the large pools."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = f32_to_bf16_bits(x) if dtype == BF16 else x
    return out.reshape(shape)


def _poison_value(dtype: str):
    return BF16_NAN_BITS if dtype == BF16 else np.float32(np.nan)


def live_slot_mask(page_table: np.ndarray, seq_lens: np.ndarray, num_pages: int,
                   page_size: int) -> np.ndarray:
    """bool [NP, P]: True where a (page, slot) holds a key some request reads."""
    live = np.zeros((num_pages, page_size), dtype=bool)
    for r in range(seq_lens.size):
        L = int(seq_lens[r])
        npg = (L + page_size - 1) // page_size
        for k in range(npg):
            n = min(page_size, L - k * page_size)
            live[page_table[r, k], :n] = True
    return live


def make_batch(name: str, seed: int, seq_lens, q_offsets, num_q_heads: int, num_kv_heads: int,
               head_dim: int, page_size: int = 16, dtype: str = BF16, pool: str = "permuted",
               pool_factor: float = 1.25, num_pages: Optional[int] = None,
               poison: bool = True, num_splits: Optional[int] = None,
               rng: Optional[np.random.Generator] = None, zero_values: bool = False) -> PagedBatch:
    """Build one batch.

    pool: "permuted"    -- pool of num_pages (default ceil(pool_factor * needed))
                           pages, assigned from a seeded permutation
          "interleaved" -- exactly the needed pages, grown round-robin
          "identity"    -- request r's pages are consecutive and in order
    poison: fill page tails and unused pages with NaN (parity runs); else 0.
    zero_values: all-zero q/K/V (used only to size timing runs quickly).
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_offsets = np.asarray(q_offsets, dtype=np.int32)
    assert seq_lens.shape == q_offsets.shape
    assert np.all(seq_lens >= 1) and np.all(q_offsets >= 0) and np.all(q_offsets < seq_lens)
    assert num_q_heads % num_kv_heads == 0
    n_pages = pages_for(seq_lens, page_size)
    needed = int(n_pages.sum())
    if pool == "permuted":
        NP = int(num_pages) if num_pages is not None else int(math.ceil(pool_factor * needed))
        table = assign_pages_permuted(rng, n_pages, NP)
    elif pool == "interleaved":
        NP = needed
        table = assign_pages_interleaved(n_pages)
    elif pool == "identity":
        NP = int(num_pages) if num_pages is not None else needed
        mp = int(n_pages.max())
        table = np.full((seq_lens.size, mp), -1, dtype=np.int32)
        pos = 0
        for r, n in enumerate(n_pages):
            table[r, :n] = np.arange(pos, pos + n, dtype=np.int32)
            pos += n
    else:
        raise ValueError(pool)

    total_q = int((seq_lens - q_offsets).sum())
    pool_shape = (NP, num_kv_heads, page_size, head_dim)
    q_shape = (total_q, num_q_heads, head_dim)
    if zero_values:
        st = np.uint16 if dtype == BF16 else np.float32
        q = np.zeros(q_shape, st)
        k_pool = np.zeros(pool_shape, st)
        v_pool = np.zeros(pool_shape, st)
    else:
        q = _normal(rng, q_shape, dtype)
        k_pool = _normal(rng, pool_shape, dtype)
        v_pool = _normal(rng, pool_shape, dtype)
    live = live_slot_mask(table, seq_lens, NP, page_size)
    dead = ~live
    if dead.any():
        fill = _poison_value(dtype) if poison else (np.uint16(0) if dtype == BF16 else np.float32(0))
        # broadcast the (page, slot) mask over heads and dims
        k_pool.transpose(0, 2, 1, 3)[dead] = fill
        v_pool.transpose(0, 2, 1, 3)[dead] = fill
    return PagedBatch(name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
                      num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                      seq_lens=seq_lens, q_offsets=q_offsets, page_table=table,
                      k_pool=k_pool, v_pool=v_pool, q=q, scale=1.0 / math.sqrt(head_dim),
                      num_splits=num_splits, notes={"pool": pool, "poison": poison})


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------
CONFIG_NAMES = ("tiny_decode", "qwen3_0p6b_decode", "qwen3_4b_decode", "mixed_step",
                "long_splitk_decode")

CONFIG_DOC = {
    "tiny_decode": "2 requests, contexts 37 and 100, 4 q heads / 2 KV heads, d=64, P=16, "
                   "16-page pool assigned by a seeded permutation, fp32, one query token each",
    "qwen3_0p6b_decode": "batch 32, 16/8 heads, d=128, bf16, P=16, contexts U[128,2048], "
                         "permuted pool of 1.25x the needed pages",
    "qwen3_4b_decode": "batch 64, 32/8 heads, d=128, bf16, P=16, contexts U[1024,8192], "
                       "fragmented pool grown round-robin across requests",
    "mixed_step": "4 prefill chunks of 512 tokens at offsets {0,512,1536,3072} plus 60 decode "
                  "rows with contexts U[256,4096]; 32/8 heads, d=128, bf16, P=16, permuted pool "
                  "of 1.25x",
    "long_splitk_decode": "batch 16, 32/8 heads, d=64, bf16, P=16, context 32768 each, 16 splits, "
                          "pool of exactly the needed pages, permuted",
}

DEFAULT_SEEDS = {n: i for i, n in enumerate(CONFIG_NAMES)}


def make_config(name: str, seed: Optional[int] = None, poison: bool = True,
                zero_values: bool = False) -> PagedBatch:
    if isinstance(name, int):
        name = CONFIG_NAMES[name]
    seed = DEFAULT_SEEDS[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    kw = dict(poison=poison, rng=rng, zero_values=zero_values)
    if name == "tiny_decode":
        L = np.array([37, 100], np.int32)
        return make_batch(name, seed, L, L - 1, 4, 2, 64, 16, F32, pool="permuted",
                          num_pages=16, **kw)
    if name == "qwen3_0p6b_decode":
        L = rng.integers(128, 2048 + 1, size=32).astype(np.int32)
        return make_batch(name, seed, L, L - 1, 16, 8, 128, 16, BF16, pool="permuted",
                          pool_factor=1.25, **kw)
    if name == "qwen3_4b_decode":
        L = rng.integers(1024, 8192 + 1, size=64).astype(np.int32)
        return make_batch(name, seed, L, L - 1, 32, 8, 128, 16, BF16, pool="interleaved", **kw)
    if name == "mixed_step":
        o_pf = np.array([0, 512, 1536, 3072], np.int32)
        L_pf = o_pf + 512
        L_dec = rng.integers(256, 4096 + 1, size=60).astype(np.int32)
        L = np.concatenate([L_pf, L_dec])
        o = np.concatenate([o_pf, L_dec - 1])
        b = make_batch(name, seed, L, o, 32, 8, 128, 16, BF16, pool="permuted",
                       pool_factor=1.25, **kw)
        b.notes["prefill_requests"] = (0, 4)
        b.notes["decode_requests"] = (4, 64)
        return b
    if name == "long_splitk_decode":
        L = np.full(16, 32768, np.int32)
        return make_batch(name, seed, L, L - 1, 32, 8, 64, 16, BF16, pool="permuted",
                          pool_factor=1.0, num_splits=16, **kw)
    raise KeyError(name)
