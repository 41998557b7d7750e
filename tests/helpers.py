"""Shared test plumbing: moving a seeded batch to the GPU, running the oracle
on it, and comparing results.  Nothing here computes attention."""
from __future__ import annotations

import numpy as np
import torch

import oracle as ORACLE
import workloads as W

OUT_TOL_BF16 = 1e-2      # max |out_gpu - out_oracle|, bf16 I/O, fp32 accumulation
LSE_TOL = 1e-3           # max |lse_gpu - lse_oracle|
OUT_TOL_F32 = 1e-5       # fp32 I/O (tiny config): float32 end to end
LSE_TOL_F32 = 1e-5


def to_torch(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == W.BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def device_batch(b: W.PagedBatch, device="cuda") -> dict:
    return {
        "q": to_torch(b.q, b.dtype, device),
        "k_pool": to_torch(b.k_pool, b.dtype, device),
        "v_pool": to_torch(b.v_pool, b.dtype, device),
        "page_table": torch.from_numpy(np.ascontiguousarray(b.page_table)).to(device),
        "seq_lens": torch.from_numpy(np.ascontiguousarray(b.seq_lens)).to(device),
        "q_offsets": torch.from_numpy(np.ascontiguousarray(b.q_offsets)).to(device),
    }


def oracle_run(b: W.PagedBatch, requests=None):
    return ORACLE.paged_attention(b.q_f32(), b.k_pool_f32(), b.v_pool_f32(), b.page_table,
                                  b.seq_lens, b.q_offsets, b.scale, requests=requests)


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rne_bf16_f64(x: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)


# Stress inputs (scores scaled far beyond N(0,1)) drive the output towards a
# single value row, so |out| can exceed 2, where one bf16 rounding step of the
# output alone is >= 2^-8 |out|.  Those tests add this relative term to the
# absolute bar; the named workloads use the absolute bar alone.
STRESS_REL = 2.0 ** -8


def compare(b: W.PagedBatch, out: torch.Tensor, lse: torch.Tensor, ref_out, ref_lse, rows=None,
            label="", rel=0.0):
    """Element-wise comparison against the oracle; returns a stats dict and
    asserts the tolerance for the batch's dtype (|d out| <= tol + rel*|ref|)."""
    o = out_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o, l, ref_out, ref_lse = o[rows], l[rows], ref_out[rows], ref_lse[rows]
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    assert np.all(np.isfinite(l)), f"{label}: non-finite lse"
    d_out = np.abs(o - ref_out)
    d_lse = np.abs(l - ref_lse)
    stats = {"max_abs_out_err": float(d_out.max()), "max_abs_lse_err": float(d_lse.max()),
             "max_abs_oracle_out": float(np.abs(ref_out).max())}
    excess = float((d_out - rel * np.abs(ref_out)).max())
    if b.dtype == W.BF16:
        ulp = np.abs(o - rne_bf16_f64(ref_out))
        stats["max_abs_vs_rne_oracle"] = float(ulp.max())
        tol_o, tol_l = OUT_TOL_BF16, LSE_TOL
    else:
        tol_o, tol_l = OUT_TOL_F32, LSE_TOL_F32
    print(f"[{label}] {stats}", flush=True)
    assert excess <= tol_o, (label, stats)
    assert stats["max_abs_lse_err"] <= tol_l, (label, stats)
    return stats
