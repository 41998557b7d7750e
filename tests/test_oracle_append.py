"""Pins for the KV-append oracle (oracle/kv_append.py).

Each pin checks the append against something other than itself: reading the
appended positions back through the gather (pinned separately by the
hand-written page-table fixture), the dense view of a pool whose page table
is the identity, and the slots no new row maps to.  As for the attention
oracle, every pin takes the module under test as an argument so that planted
mistakes can be run through the same pins.
"""
import os
import types

import numpy as np
import pytest

import oracle as ORACLE
from oracle import kv_append as KVA


def _case(seed, lens, offs, Hkv=3, d=8, P=4, identity=False, pool_factor=2.0, dtype=np.float32):
    rng = np.random.default_rng(seed)
    lens = np.array(lens, np.int32)
    offs = np.array(offs, np.int32)
    npg = (lens + P - 1) // P
    MP = int(npg.max())
    if identity:
        NP = int(npg.sum())
        ids = np.arange(NP, dtype=np.int32)
    else:
        NP = int(np.ceil(pool_factor * npg.sum()))
        ids = rng.permutation(NP).astype(np.int32)
    table = np.full((len(lens), MP), -1, np.int32)
    at = 0
    for r, n in enumerate(npg):
        table[r, :n] = ids[at:at + n]
        at += n
    if dtype == np.uint16:   # raw bf16 bit patterns, NaN payloads included
        kp = rng.integers(0, 1 << 16, size=(NP, Hkv, P, d), dtype=np.uint16)
        vp = rng.integers(0, 1 << 16, size=(NP, Hkv, P, d), dtype=np.uint16)
    else:
        kp = rng.standard_normal((NP, Hkv, P, d)).astype(dtype)
        vp = rng.standard_normal((NP, Hkv, P, d)).astype(dtype)
    rows = int((lens - offs).sum())
    if dtype == np.uint16:
        kn = rng.integers(0, 1 << 16, size=(rows, Hkv, d), dtype=np.uint16)
        vn = rng.integers(0, 1 << 16, size=(rows, Hkv, d), dtype=np.uint16)
    else:
        kn = (rng.standard_normal((rows, Hkv, d)) + 100.0).astype(dtype)   # distinct from the pool
        vn = (rng.standard_normal((rows, Hkv, d)) - 100.0).astype(dtype)
    return kp, vp, table, lens, offs, kn, vn


CASES = [
    dict(seed=1, lens=[5, 9, 1], offs=[0, 8, 0]),        # full prompt, one decode token, single key
    dict(seed=2, lens=[12, 7, 16], offs=[3, 4, 15]),     # chunks crossing page boundaries
    dict(seed=3, lens=[4, 8], offs=[0, 4]),              # page-aligned chunks
]


def pin_gather_roundtrip(mod):
    for c in CASES:
        kp, vp, table, lens, offs, kn, vn = _case(**c)
        k2, v2 = mod.append_kv(kp, vp, table, lens, offs, kn, vn)
        row = 0
        for r in range(len(lens)):
            K, V = ORACLE.gather(k2, v2, table[r], int(lens[r]))
            n = int(lens[r] - offs[r])
            assert np.array_equal(K[offs[r]:lens[r]], kn[row:row + n])
            assert np.array_equal(V[offs[r]:lens[r]], vn[row:row + n])
            row += n


def pin_identity_is_dense(mod):
    for c in CASES:
        kp, vp, table, lens, offs, kn, vn = _case(**c, identity=True)
        k2, v2 = mod.append_kv(kp, vp, table, lens, offs, kn, vn)
        P = kp.shape[2]
        row = 0
        for r in range(len(lens)):
            first = int(table[r, 0])
            npg = (int(lens[r]) + P - 1) // P
            # the request's pages are consecutive: its cache is a reshape of a slice
            dense_k = k2[first:first + npg].transpose(0, 2, 1, 3).reshape(npg * P, kp.shape[1], -1)
            dense_v = v2[first:first + npg].transpose(0, 2, 1, 3).reshape(npg * P, kp.shape[1], -1)
            n = int(lens[r] - offs[r])
            assert np.array_equal(dense_k[offs[r]:lens[r]], kn[row:row + n])
            assert np.array_equal(dense_v[offs[r]:lens[r]], vn[row:row + n])
            row += n


def pin_other_slots_untouched(mod):
    for c in CASES:
        kp, vp, table, lens, offs, kn, vn = _case(**c)
        k2, v2 = mod.append_kv(kp, vp, table, lens, offs, kn, vn)
        P = kp.shape[2]
        written = set()
        for r in range(len(lens)):
            for pos in range(int(offs[r]), int(lens[r])):
                written.add((int(table[r, pos // P]), pos % P))
        for page in range(kp.shape[0]):
            for slot in range(P):
                if (page, slot) not in written:
                    assert np.array_equal(k2[page, :, slot], kp[page, :, slot])
                    assert np.array_equal(v2[page, :, slot], vp[page, :, slot])
        # the inputs themselves are not modified
        kp0, vp0, *_ = _case(**c)
        assert np.array_equal(kp, kp0) and np.array_equal(vp, vp0)


def pin_bits_are_copied(mod):
    kp, vp, table, lens, offs, kn, vn = _case(seed=9, lens=[13, 6], offs=[2, 0], dtype=np.uint16)
    k2, v2 = mod.append_kv(kp, vp, table, lens, offs, kn, vn)
    assert k2.dtype == np.uint16 and v2.dtype == np.uint16
    K, V = ORACLE.gather(k2, v2, table[0], 13)
    assert np.array_equal(K[2:13].view(np.uint8), kn[:11].view(np.uint8))
    assert np.array_equal(V[2:13].view(np.uint8), vn[:11].view(np.uint8))


PINS = [pin_gather_roundtrip, pin_identity_is_dense, pin_other_slots_untouched, pin_bits_are_copied]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(KVA)


MUTANTS = {
    "slot_shifted": ("slot = pos % P", "slot = (pos + 1) % P"),
    "page_from_slot": ("page = int(page_table[r][pos // P])", "page = int(page_table[r][pos % P])"),
    "row_off_by_one": ("k_out[page, :, slot, :] = k_new[row]", "k_out[page, :, slot, :] = k_new[row - 1]"),
    "v_from_k": ("v_out[page, :, slot, :] = v_new[row]", "v_out[page, :, slot, :] = k_new[row]"),
    "positions_shifted": ("for pos in range(int(q_offsets[r]), int(seq_lens[r])):",
                          "for pos in range(int(q_offsets[r]) + 1, int(seq_lens[r]) + 1):"),
    "heads_reversed": ("k_out[page, :, slot, :] = k_new[row]", "k_out[page, :, slot, :] = k_new[row][::-1]"),
    "in_place": ("k_out = k_pool.copy()", "k_out = k_pool"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name):
    src = open(KVA.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, old
    mod = types.ModuleType("kv_append_mutant")
    exec(compile(src.replace(old, new, 1), "kv_append_mutant", "exec"), mod.__dict__)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:   # assertion or crash both count as caught
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


# ---- copy_pages (the device half of a copy on write) ----

def _copy_case(seed):
    rng = np.random.default_rng(seed)
    NP, Hkv, P, d = 12, 3, 4, 8
    kp = rng.standard_normal((NP, Hkv, P, d)).astype(np.float32)
    vp = rng.standard_normal((NP, Hkv, P, d)).astype(np.float32)
    src = np.array([3, 7, 0], np.int32)
    dst = np.array([10, 2, 5], np.int32)
    return kp, vp, src, dst


def cpin_gather_through_copy(mod):
    kp, vp, src, dst = _copy_case(21)
    k2, v2 = mod.copy_pages(kp, vp, src, dst)
    P = kp.shape[2]
    # a request whose table names the source pages, and the same request
    # with the copies in their place, gather the same keys and values
    t_src = np.array(src, np.int32)
    t_dst = np.array(dst, np.int32)
    L = len(src) * P - 1
    Ks, Vs = ORACLE.gather(k2, v2, t_src, L)
    Kd, Vd = ORACLE.gather(k2, v2, t_dst, L)
    assert np.array_equal(Ks, Kd) and np.array_equal(Vs, Vd)
    K0, V0 = ORACLE.gather(kp, vp, t_src, L)
    assert np.array_equal(Kd, K0) and np.array_equal(Vd, V0)


def cpin_other_pages_untouched(mod):
    kp, vp, src, dst = _copy_case(22)
    k2, v2 = mod.copy_pages(kp, vp, src, dst)
    for page in range(kp.shape[0]):
        if page not in dst:
            assert np.array_equal(k2[page], kp[page]) and np.array_equal(v2[page], vp[page])
    kp0, vp0, *_ = _copy_case(22)
    assert np.array_equal(kp, kp0) and np.array_equal(vp, vp0)


def cpin_bad_pairs_are_skipped(mod):
    kp, vp, _, _ = _copy_case(23)
    k2, v2 = mod.copy_pages(kp, vp, np.array([4, -1, 99, 6], np.int32), np.array([4, 2, 3, -5], np.int32))
    assert np.array_equal(k2, kp) and np.array_equal(v2, vp)


CPINS = [cpin_gather_through_copy, cpin_other_pages_untouched, cpin_bad_pairs_are_skipped]


@pytest.mark.parametrize("pin", CPINS, ids=lambda p: p.__name__)
def test_copy_pin(pin):
    pin(KVA)


COPY_MUTANTS = {
    "direction_swapped": ("k_out[d_id] = k_pool[s_id]", "k_out[s_id] = k_pool[d_id]"),
    "v_from_k": ("v_out[d_id] = v_pool[s_id]", "v_out[d_id] = k_pool[s_id]"),
    "one_head_only": ("k_out[d_id] = k_pool[s_id]", "k_out[d_id, 0] = k_pool[s_id, 0]"),
    "no_skip_checks": ("if not (0 <= s_id < num_pages and 0 <= d_id < num_pages) or s_id == d_id:",
                       "if False:"),
    "in_place": ("k_out = k_pool.copy()\n    v_out = v_pool.copy()\n    num_pages",
                 "k_out = k_pool\n    v_out = v_pool.copy()\n    num_pages"),
}


@pytest.mark.parametrize("name", sorted(COPY_MUTANTS))
def test_copy_mutants_are_caught(name):
    src = open(KVA.__file__).read()
    old, new = COPY_MUTANTS[name]
    assert src.count(old) >= 1, old
    mod = types.ModuleType("kv_copy_mutant")
    exec(compile(src.replace(old, new, 1), "kv_copy_mutant", "exec"), mod.__dict__)
    caught = []
    for pin in CPINS:
        try:
            pin(mod)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
