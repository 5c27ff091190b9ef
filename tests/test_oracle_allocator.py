"""CPU pins of the allocator oracle: the pages' worked examples and invariants."""
import numpy as np
import pytest

from oracle import allocator as AL
from tests import oracle_pins as P


def test_p1_block_mapping_example():
    P.check_p1_block_mapping()


def test_block_counts_examples():
    P.check_block_counts()


def test_addressing_example():
    P.check_addressing()


def test_cow_timeline():
    P.check_p4_cow_timeline()


def test_refcount_lifecycle():
    P.check_p2_lifecycle()


def test_exhaustion_leaves_state_unchanged():
    al = AL.BlockAllocator(3, 16)
    al.seq_create(1, 32)
    al.seq_fork(1, 2)
    before = al.clone()
    with pytest.raises(AL.AllocatorError) as e:
        al.seq_create(3, 40)
    assert e.value.code == AL.NO_FREE_BLOCKS
    al.seq_append_slot(1)          # 32 % 16 == 0: takes the last free block
    snap = al.clone()
    with pytest.raises(AL.AllocatorError):
        al.seq_append_slot(2)      # needs another fresh block: none left
    assert al.free_list() == snap.free_list() and al.refs == snap.refs
    assert al.tables == snap.tables and al.lens == snap.lens
    # a batch that fails half-way is rolled back whole
    al2 = before.clone()
    with pytest.raises(AL.AllocatorError):
        al2.seq_append_slots([1, 2])
    assert al2.tables == before.tables and al2.refs == before.refs and al2.free_list() == before.free_list()


def test_errors():
    al = AL.BlockAllocator(4, 16)
    al.seq_create(1, 5)
    with pytest.raises(AL.AllocatorError) as e:
        al.seq_create(1, 5)
    assert e.value.code == AL.SEQ_EXISTS
    with pytest.raises(AL.AllocatorError) as e:
        al.seq_free(9)
    assert e.value.code == AL.UNKNOWN_SEQ
    with pytest.raises(AL.AllocatorError) as e:
        al.seq_fork(1, 2, 6)
    assert e.value.code == AL.INVALID_ARG
    with pytest.raises(AL.AllocatorError):
        AL.BlockAllocator(3, 16, initial_free_order=[0, 0, 1])
    assert al.ref_count(-1) == -1 and al.ref_count(4) == -1


def test_append_crosses_blocks_and_cow_once_per_sharer():
    al = AL.BlockAllocator(16, 4)
    al.seq_create(0, 6)                # blocks [0, 1], block 1 half full
    for c in (1, 2, 3):
        al.seq_fork(0, c)
    assert al.ref_count(1) == 4
    res = [al.seq_append_slot(s) for s in (0, 1, 2, 3)]
    # the first three writers copy, the last finds itself sole owner and writes in place
    assert [r[1:] for r in res] == [(1, 2), (1, 3), (1, 4), (-1, -1)]
    assert al.block_table(3) == [0, 1] and al.ref_count(1) == 1
    assert [r[0] for r in res] == [2 * 4 + 2, 3 * 4 + 2, 4 * 4 + 2, 1 * 4 + 2]
    assert al.ref_count(0) == 4


def test_random_operations_keep_pool_invariants():
    rng = np.random.default_rng(0)
    al = AL.BlockAllocator(64, 8, initial_free_order=rng.permutation(64))
    live = []
    nxt = 0
    for _ in range(3000):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                al.seq_create(nxt, int(rng.integers(0, 40)))
                live.append(nxt)
                nxt += 1
            elif op == 1:
                p = live[rng.integers(len(live))]
                al.seq_fork(p, nxt, int(rng.integers(-1, al.seq_len(p) + 1)))
                live.append(nxt)
                nxt += 1
            elif op == 2:
                al.seq_append_slots([live[i] for i in rng.integers(0, len(live), size=3)])
            else:
                al.seq_free(live.pop(rng.integers(len(live))))
        except AL.AllocatorError as e:
            assert e.code == AL.NO_FREE_BLOCKS
        # every block is either free (count 0) or referenced exactly count times
        counts = np.zeros(64, dtype=int)
        for t in al.tables.values():
            for b in t:
                counts[b] += 1
        assert list(counts) == al.refs
        assert sorted(al.free_list()) == [b for b in range(64) if counts[b] == 0]
        for s, t in al.tables.items():
            assert len(t) == -(-al.lens[s] // 8)
