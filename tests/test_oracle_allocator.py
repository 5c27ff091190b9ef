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


def test_p4_prefix_demo():
    P.check_p4_prefix_demo()


def test_prefix_random_operations_keep_pool_invariants():
    """Random prefix, sequence and append operations: every block's count equals the
    references held by sequences and prefix entries; sequences built on a prefix start
    with its blocks and never get a copy-on-write pair for them."""
    rng = np.random.default_rng(4)
    NB, bs = 96, 8
    al = AL.BlockAllocator(NB, bs, initial_free_order=rng.permutation(NB))
    prompts = [list(rng.integers(0, 50, size=int(n))) for n in (0, 3, 8, 11, 16, 21)]
    live, users, nxt = [], [], 0
    for _ in range(3000):
        op = int(rng.integers(0, 7))
        try:
            if op == 0:
                pid, _ = al.prefix_get_or_create(prompts[int(rng.integers(len(prompts)))])
                users.append(pid)
            elif op == 1 and users:
                pid = users[int(rng.integers(len(users)))]
                al.seq_create_with_prefix(nxt, pid, int(rng.integers(0, 20)))
                live.append(nxt)
                nxt += 1
            elif op == 2 and users:
                al.prefix_release(users.pop(int(rng.integers(len(users)))))
            elif op == 3 and live:
                p = live[int(rng.integers(len(live)))]
                al.seq_fork(p, nxt, int(rng.integers(-1, al.seq_len(p) + 1)))
                live.append(nxt)
                nxt += 1
            elif op == 4 and live:
                _, pairs = al.seq_append_slots([live[i] for i in rng.integers(0, len(live), size=3)])
                entry_blocks = {b for e in al.entries.values() for b in e["blocks"]}
                assert not [p for p in pairs if p[0] in entry_blocks and al.holes]
            elif op == 5 and live:
                al.seq_free(live.pop(int(rng.integers(len(live)))))
            else:
                al.seq_create(nxt, int(rng.integers(0, 30)))
                live.append(nxt)
                nxt += 1
        except AL.AllocatorError as e:
            assert e.code in (AL.NO_FREE_BLOCKS, AL.INVALID_ARG)
        counts = np.zeros(NB, dtype=int)
        for t in al.tables.values():
            for b in t:
                counts[b] += 1
        for e in al.entries.values():
            for b in e["blocks"]:
                counts[b] += 1
        assert list(counts) == al.refs
        assert sorted(al.free_list()) == [b for b in range(NB) if counts[b] == 0]
        for s, (lo, hi) in al.holes.items():
            assert lo < hi <= al.lens[s] and hi % bs == 0
        assert sum(e["users"] for e in al.entries.values()) == len(users)


@pytest.mark.parametrize("pin", P.SWAP_WINDOW_PINS, ids=[p.__name__ for p in P.SWAP_WINDOW_PINS])
def test_swap_window_pin(pin):
    pin()
