"""Why the prefill P V product keeps more than bf16 precision in its weights.

A CPU model of the kernel's rounding steps, checked against the fp64 oracle:
the chunk's 128-row tiles, their key range split in two halves, 64-key
steps with the lazy running max (moved only when a score exceeds it by more
than 2^8 in base 2), weights p = 2^(s*scale*log2 e - m) in fp32, the row sum
from the fp32 weights, and the output rounded to bf16.  The only knob is how
the weights enter the P V product: rounded to bf16 (8-bit significand), to
fp16 (11 bits; the kernel's choice) or as a bf16 pair (high part plus
remainder).  On rows dominated by a few values near 4 the bf16 weights move
outputs past the 1e-2 bar; fp16 weights and the pair stay inside it.

A fourth form keeps bf16 weights but divides by the sum of the rounded
weights (so the weights' rounding errors cancel against v - o instead of
adding up): closer, still past the bar, because near |o| = 4 the output's
own bf16 rounding takes up to 2^-7 of it and leaves about 2e-3 for the
weights, which needs fp16's 11 bits.  CPU only; the GPU tests check the
kernel itself on the same case."""
import math

import numpy as np
import pytest

import oracle as ORACLE
import workloads as W

OUT_TOL = 1e-2


def bf16(x):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.asarray(x, np.float32)))


def weights_as(p, mode):
    if mode in ("bf16", "bf16_self"):
        return bf16(p).astype(np.float64)
    if mode == "f16":
        return p.astype(np.float16).astype(np.float64)
    hi = bf16(p)
    return hi.astype(np.float64) + bf16(p - hi)


def model_request(q, K, V, o, G, scale, mode):
    """One request's (KV head's) rows, packed token-major, as the kernel
    forms them; returns bf16 outputs (as float64).  Mode "bf16_self" rounds
    the weights to bf16 and sums the rounded weights for the divisor; every
    other mode sums the fp32 weights."""
    n, _, d = q.shape
    rows = n * G
    Q = q.reshape(rows, d).astype(np.float64)
    pos = o + np.arange(rows) // G
    sl2 = np.float32(scale * math.log2(math.e))
    S = (Q @ K.astype(np.float64).T).astype(np.float32)
    out = np.zeros((rows, d))
    for rb in range(0, rows, 128):
        r1 = min(rows, rb + 128)
        kmax = o + (r1 - 1) // G + 1
        nt = (kmax + 63) // 64
        mid = (nt + 1) // 2
        parts = []
        for lo, hi in ((0, mid), (mid, nt)):
            R = r1 - rb
            m = np.full(R, -np.inf, np.float32)
            l = np.zeros(R, np.float32)
            acc = np.zeros((R, d))
            for kt in range(lo, hi):
                k0, k1 = kt * 64, min(kt * 64 + 64, kmax)
                vis = np.arange(k0, k1)[None, :] <= pos[rb:r1, None]
                s = np.where(vis, S[rb:r1, k0:k1], -np.inf)
                tmax = (s.max(axis=1) * sl2).astype(np.float32)
                need = tmax > m + 8
                if need.any():
                    mn = np.maximum(m, tmax)
                    alpha = np.where(np.isneginf(m), 0.0, np.exp2((m - mn).astype(np.float64)))
                    l = np.where(need, l * alpha, l).astype(np.float32)
                    acc = np.where(need[:, None], acc * alpha[:, None], acc)
                    m = np.where(need, mn, m)
                mref = np.where(np.isneginf(m), 0, m).astype(np.float32)
                p = np.where(vis, np.exp2((s * sl2 - mref[:, None]).astype(np.float32)), 0).astype(np.float32)
                if mode == "bf16_self":
                    p = bf16(p).astype(np.float32)
                l = (l + p.sum(axis=1, dtype=np.float32)).astype(np.float32)
                acc = acc + weights_as(p, mode) @ V[k0:k1].astype(np.float64)
            parts.append((m, l, acc))
        (mA, lA, oA), (mB, lB, oB) = parts
        M = np.maximum(mA, mB)
        fA = np.where(np.isneginf(mA), 0, np.exp2(mA - M))
        fB = np.where(np.isneginf(mB), 0, np.exp2(mB - M))
        out[rb:r1] = (oA * fA[:, None] + oB * fB[:, None]) / (lA * fA + lB * fB)[:, None]
    return bf16(out).astype(np.float64)


def few_dominant_keys_case(seed):
    # the GPU test's case (tests/test_gpu_prefill.py), at 2 of its 8 KV heads
    b = W.make_batch("few dominant keys", seed, np.array([512], np.int32), np.array([0], np.int32),
                     8, 2, 128, 16, W.BF16)
    b.q = W.f32_to_bf16_bits(b.q_f32() * 4.0)
    vp = b.v_pool_f32().copy()
    for pg in b.page_table[0, :2]:
        x = vp[pg]
        vp[pg] = np.sign(x) * (3.0 + 0.875 * np.abs(np.tanh(x)))
    b.v_pool = W.f32_to_bf16_bits(np.clip(vp, -3.875, 3.875))
    return b


def max_err(b, mode):
    ref, _ = ORACLE.paged_attention(b.q_f32(), b.k_pool_f32(), b.v_pool_f32(), b.page_table,
                                    b.seq_lens, b.q_offsets, b.scale)
    G = b.num_q_heads // b.num_kv_heads
    K, V = ORACLE.gather(b.k_pool_f32(), b.v_pool_f32(), b.page_table[0], int(b.seq_lens[0]))
    q = b.q_f32()
    err = 0.0
    for g in range(b.num_kv_heads):
        o = model_request(q[:, g * G:(g + 1) * G], K[:, g], V[:, g], 0, G, b.scale, mode)
        err = max(err, float(np.abs(o.reshape(ref[:, g * G:(g + 1) * G].shape) -
                                    ref[:, g * G:(g + 1) * G]).max()))
    return err, float(np.abs(ref).max())


@pytest.mark.parametrize("seed", [100, 101])
def test_bf16_weights_cross_the_bar_where_fp16_weights_do_not(seed):
    b = few_dominant_keys_case(seed)
    e_bf16, omax = max_err(b, "bf16")
    e_f16, _ = max_err(b, "f16")
    e_pair, _ = max_err(b, "pair")
    e_self, _ = max_err(b, "bf16_self")
    print(f"seed {seed}: max|out| {omax:.3f}; max|d out| bf16 {e_bf16:.4f}, fp16 {e_f16:.4f}, "
          f"bf16 pair {e_pair:.4f}, bf16 over its own sum {e_self:.4f}")
    assert omax < 4.0                 # the range where the 1e-2 bar leaves room for one bf16 step
    assert e_bf16 > OUT_TOL           # one bf16 rounding of the weights is not enough
    assert e_self > OUT_TOL           # ... even when the divisor sums the same rounded weights
    assert e_self < e_bf16
    assert e_f16 <= OUT_TOL and e_pair <= OUT_TOL
