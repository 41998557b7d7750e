"""Host page allocator (pa_pool_*): pure host logic, no GPU."""
import numpy as np
import pytest

import paged_kv_cache_02_amd as pa


def test_alloc_hands_out_distinct_ids_in_range_until_exhausted():
    pool = pa.PagePool(10)
    a = pool.alloc(4)
    b = pool.alloc(6)
    ids = np.concatenate([a, b])
    assert sorted(ids.tolist()) == list(range(10))
    assert pool.num_free == 0
    with pytest.raises(pa.PaError) as e:
        pool.alloc(1)
    assert e.value.code == pa.PA_ERR_NO_PAGES


def test_exhaustion_is_all_or_nothing():
    pool = pa.PagePool(5)
    pool.alloc(3)
    with pytest.raises(pa.PaError):
        pool.alloc(3)
    assert pool.num_free == 2
    assert len(pool.alloc(2)) == 2


def test_free_returns_pages_and_rejects_bad_ids_without_side_effects():
    pool = pa.PagePool(8)
    a = pool.alloc(5)
    pool.free(a[:2])
    assert pool.num_free == 5
    for bad in ([a[0]],            # already free
                [a[2], a[2]],      # repeated
                [99],              # out of range
                [-1],
                [a[3], 7 if 7 not in a else 6]):   # second id never allocated
        with pytest.raises(pa.PaError) as e:
            pool.free(np.array(bad, np.int32))
        assert e.value.code == pa.PA_ERR_ARG
        assert pool.num_free == 5
    pool.free(a[2:])
    assert pool.num_free == 8


def test_reserve_grows_a_row_by_whole_pages_and_release_empties_it():
    P = 16
    pool = pa.PagePool(100)
    row = np.full(8, -1, np.int32)
    pool.reserve(row, 0, 1, P)            # 1 key -> 1 page
    assert (row[:1] >= 0).all() and (row[1:] == -1).all()
    first = int(row[0])
    pool.reserve(row, 1, 16, P)           # still 1 page: nothing new
    assert row[0] == first and (row[1:] == -1).all() and pool.num_free == 99
    pool.reserve(row, 16, 17, P)          # crosses into page 2
    assert row[1] >= 0 and row[1] != first and pool.num_free == 98
    pool.reserve(row, 17, 100, P)         # up to ceil(100/16) = 7 pages
    assert (row[:7] >= 0).all() and row[7] == -1 and len(set(row[:7].tolist())) == 7
    assert pool.num_free == 93
    with pytest.raises(pa.PaError) as e:
        pool.reserve(row, 100, 200, P)    # more pages than the row holds
    assert e.value.code == pa.PA_ERR_ARG
    assert pool.num_free == 93 and row[7] == -1
    pool.release(row, 100, P)
    assert (row == -1).all() and pool.num_free == 100


def test_reserve_that_cannot_be_met_changes_nothing():
    pool = pa.PagePool(3)
    row = np.full(8, -1, np.int32)
    with pytest.raises(pa.PaError) as e:
        pool.reserve(row, 0, 64, 16)      # needs 4 pages, 3 free
    assert e.value.code == pa.PA_ERR_NO_PAGES
    assert (row == -1).all() and pool.num_free == 3


def test_many_requests_never_share_a_page():
    rng = np.random.default_rng(0)
    P, B, MP = 16, 12, 20
    pool = pa.PagePool(B * MP)
    table = np.full((B, MP), -1, np.int32)
    lens = np.zeros(B, np.int64)
    for step in range(200):
        r = int(rng.integers(B))
        if lens[r] > 0 and rng.random() < 0.1:       # request finishes
            pool.release(table[r], int(lens[r]), P)
            lens[r] = 0
            continue
        grow = int(rng.integers(1, 40))
        new = min(int(lens[r]) + grow, MP * P)
        pool.reserve(table[r], int(lens[r]), new, P)
        lens[r] = new
        used = table[table >= 0]
        assert len(set(used.tolist())) == used.size           # no page in two places
        assert pool.num_free + used.size == B * MP            # nothing lost
        need = (lens + P - 1) // P
        assert all(((table[i] >= 0).sum() == need[i]) for i in range(B))


def test_null_and_invalid_arguments():
    L = pa.lib()
    assert L.pa_pool_num_free(None) == -1
    assert L.pa_pool_alloc(None, 1, None) == pa.PA_ERR_ARG
    import ctypes
    h = ctypes.c_void_p()
    assert L.pa_pool_create(0, ctypes.byref(h)) == pa.PA_ERR_ARG
    assert L.pa_pool_create(4, None) == pa.PA_ERR_ARG


# ---- shared pages: reference counts, fork, copy on write ----

def test_shared_page_returns_to_the_pool_after_its_last_holder():
    pool = pa.PagePool(6)
    a = pool.alloc(2)
    assert pool.refcount(a[0]) == 1
    pool.share(a)                       # a second holder of both pages
    assert pool.refcount(a[0]) == 2 and pool.refcount(a[1]) == 2
    pool.free(a)
    assert pool.num_free == 4 and pool.refcount(a[0]) == 1
    pool.free(a)
    assert pool.num_free == 6 and pool.refcount(a[0]) == 0
    assert pool.refcount(99) == -1


def test_free_may_list_a_page_as_often_as_it_is_held():
    pool = pa.PagePool(4)
    a = pool.alloc(1)
    pool.share(a)
    with pytest.raises(pa.PaError):
        pool.free(np.array([a[0]] * 3, np.int32))   # held twice, listed three times
    assert pool.refcount(a[0]) == 2
    pool.free(np.array([a[0], a[0]], np.int32))
    assert pool.refcount(a[0]) == 0 and pool.num_free == 4


def test_share_rejects_free_or_out_of_range_pages_without_side_effects():
    pool = pa.PagePool(4)
    a = pool.alloc(1)
    for bad in ([a[0], 3 if a[0] != 3 else 2], [-1], [4]):
        with pytest.raises(pa.PaError) as e:
            pool.share(np.array(bad, np.int32))
        assert e.value.code == pa.PA_ERR_ARG
    assert pool.refcount(a[0]) == 1


def test_fork_shares_a_prefix_and_release_drops_one_reference():
    P, MP = 16, 8
    pool = pa.PagePool(10)
    src = np.full(MP, -1, np.int32)
    pool.reserve(src, 0, 40, P)                        # 3 pages
    dst = np.full(MP, -1, np.int32)
    pool.fork(src, dst, 40, P)
    assert np.array_equal(dst[:3], src[:3]) and (dst[3:] == -1).all()
    assert [pool.refcount(i) for i in src[:3]] == [2, 2, 2]
    assert pool.num_free == 7
    pool.release(src, 40, P)
    assert (src[:3] == -1).all() and [pool.refcount(i) for i in dst[:3]] == [1, 1, 1]
    assert pool.num_free == 7                          # still held by dst
    pool.release(dst, 40, P)
    assert pool.num_free == 10


def test_cow_copies_only_shared_pages():
    P, MP = 16, 8
    pool = pa.PagePool(10)
    a = np.full(MP, -1, np.int32)
    pool.reserve(a, 0, 40, P)
    b = np.full(MP, -1, np.int32)
    pool.fork(a, b, 40, P)
    old, new = pool.cow(b, 2)                          # b is about to append into page 2
    assert old == a[2] and new != old and b[2] == new
    assert pool.refcount(old) == 1 and pool.refcount(new) == 1
    assert np.array_equal(b[:2], a[:2])                # the full prefix pages stay shared
    same = pool.cow(b, 2)                              # now private: no further copy
    assert same == (new, new)
    old_a, new_a = pool.cow(a, 2)                      # a is again the only holder
    assert old_a == new_a == a[2]


def test_cow_without_a_free_page_changes_nothing():
    P, MP = 16, 4
    pool = pa.PagePool(3)
    a = np.full(MP, -1, np.int32)
    pool.reserve(a, 0, 48, P)                          # all 3 pages
    b = np.full(MP, -1, np.int32)
    pool.fork(a, b, 48, P)
    with pytest.raises(pa.PaError) as e:
        pool.cow(b, 1)
    assert e.value.code == pa.PA_ERR_NO_PAGES
    assert np.array_equal(a[:3], b[:3]) and pool.refcount(b[1]) == 2
    with pytest.raises(pa.PaError):
        pool.cow(b, 3)                                 # an empty entry is not a held page
