"""CPU pins of the pool-writing oracles: slot-mapping scatter and whole-block copy."""
import numpy as np
import pytest

from oracle import cache_ops as C
from tests import oracle_pins as P


def test_reshape_hand_example():
    # pools of 4 blocks x 2 KV heads, block size 4, head dim 2 (keys as rows
    # [4, 2], values as columns [2, 4]), zeros; three new tokens
    kc = np.zeros((4, 2, 4, 2), dtype=np.float32)
    vc = np.zeros((4, 2, 2, 4), dtype=np.float32)
    key = np.arange(12, dtype=np.float32).reshape(3, 2, 2) + 1
    val = -key
    kc2, vc2 = C.reshape_and_cache(key, val, kc, vc, [5, -1, 14])
    exp_k = np.zeros_like(kc)
    exp_k[1, :, 1, :] = key[0]     # slot 5 = block 1, offset 1
    exp_k[3, :, 2, :] = key[2]     # slot 14 = block 3, offset 2; slot -1 skipped
    exp_v = np.zeros_like(vc)
    exp_v[1, 0, :, 1] = [-1, -2]   # token 0, KV head 0: dims down column 1
    exp_v[1, 1, :, 1] = [-3, -4]
    exp_v[3, 0, :, 2] = [-9, -10]  # token 2, KV head 0: column 2 of block 3
    exp_v[3, 1, :, 2] = [-11, -12]
    assert np.array_equal(kc2, exp_k)
    assert np.array_equal(vc2, exp_v)
    assert np.array_equal(kc, np.zeros_like(kc)) and np.array_equal(vc, np.zeros_like(vc))  # inputs untouched


def test_reshape_keeps_bf16_bits():
    kc = np.zeros((2, 1, 16, 4), dtype=np.uint16)
    key = np.array([[[0x7FC1, 0x0001, 0x8000, 0xFFFF]]], dtype=np.uint16)
    vc = np.zeros((2, 1, 4, 16), dtype=np.uint16)
    kc2, vc2 = C.reshape_and_cache(key, key, kc, vc, [17])
    assert np.array_equal(kc2[1, 0, 1], key[0, 0])
    assert np.array_equal(vc2[1, 0, :, 1], key[0, 0])


def test_copy_blocks_hand_example():
    kc = np.arange(4 * 2 * 2 * 2, dtype=np.float32).reshape(4, 2, 2, 2)
    vc = -kc
    kc2, vc2 = C.copy_blocks(kc, vc, [[0, 2], [1, 3]])
    assert np.array_equal(kc2[2], kc[0]) and np.array_equal(kc2[3], kc[1])
    assert np.array_equal(kc2[:2], kc[:2])
    assert np.array_equal(vc2[2], vc[0]) and np.array_equal(vc2[3], vc[1])


def test_cow_timeline_from_impl_page():
    P.check_p4_cow_timeline()


def test_swap_blocks_pin():
    P.check_swap_blocks()


def test_swap_blocks_mutants_are_caught(monkeypatch):
    """A swap that copies only the keys, or applies the pairs reversed, fails the pin."""
    from oracle import cache_ops as C

    def keys_only(dk, dv, sk, sv, pairs, _orig=C.swap_blocks):
        kd, _ = _orig(dk, dv, sk, sv, pairs)
        return kd, np.array(dv, copy=True)

    def reversed_pairs(dk, dv, sk, sv, pairs, _orig=C.swap_blocks):
        return _orig(dk, dv, sk, sv, [(b, a) for a, b in np.asarray(pairs).reshape(-1, 2).tolist()])

    for bad in (keys_only, reversed_pairs):
        monkeypatch.setattr(C, "swap_blocks", bad)
        with pytest.raises((AssertionError, IndexError)):
            P.check_swap_blocks()
