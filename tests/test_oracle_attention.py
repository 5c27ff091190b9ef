"""CPU pins of the attention oracle (closed forms, invariants, independent library)."""
import numpy as np
import pytest

from oracle import attention as A
from tests import oracle_pins as P


@pytest.mark.parametrize("S,H,Hkv,D,bs,ctx,dtype", [
    (4, 4, 4, 64, 16, (1, 16, 17, 45), "f32"),
    (3, 8, 2, 64, 16, (1, 37, 80), "f32"),
    (2, 8, 8, 128, 16, (100, 257), "f16"),
    (3, 32, 8, 128, 32, (33, 64, 130), "bf16"),
    (2, 16, 2, 64, 32, (31, 96), "f16"),
    (2, 8, 1, 64, 16, (50, 3), "bf16"),
])
def test_oracle_matches_independent_sdpa(S, H, Hkv, D, bs, ctx, dtype):
    P.check_against_sdpa(seed=S * 100 + D, S=S, H=H, Hkv=Hkv, D=D, bs=bs, ctx=ctx, dtype=dtype)


def test_brute_force_softmax():
    P.check_brute_force()


def test_two_token_closed_form():
    P.check_two_token_closed_form()


def test_identical_keys_give_mean_of_v():
    P.check_identical_keys_mean()


def test_zero_query_gives_mean_of_v():
    rng = np.random.default_rng(2)
    K, V = rng.standard_normal((33, 16)), rng.standard_normal((33, 16))
    out = A.attend(np.zeros(16), K, V, 0.25)
    assert np.max(np.abs(out - V.mean(axis=0))) <= 1e-14


def test_single_token_context_returns_v0_exactly():
    P.check_ctx1_is_v0()


def test_empty_context_gives_zeros():
    q = np.ones((1, 2, 8), dtype=np.float32)
    kc = np.ones((2, 2, 16, 8), dtype=np.float32)
    vc = np.ones((2, 2, 8, 16), dtype=np.float32)
    out = A.paged_decode(q, kc, vc, np.array([[-1]], dtype=np.int32), [0], 0.3, "f32")
    assert np.array_equal(out, np.zeros((1, 2, 8)))


def test_dominant_key_takes_all_weight():
    P.check_dominant_key()


def test_physical_block_permutation_is_bit_identical():
    P.check_permutation_invariance()


def test_key_shift_invariance():
    P.check_key_shift_invariance()


def test_value_affine_equivariance():
    P.check_value_affine()


def test_split_partials_merge_to_direct_result():
    P.check_split_merge()


def test_gather_follows_impl_page_demo():
    P.check_p4_gather_demo()


def test_scale_is_taken_at_float32():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 64)).astype(np.float32)
    kc = rng.standard_normal((2, 1, 16, 64)).astype(np.float32)
    vc = rng.standard_normal((2, 1, 64, 16)).astype(np.float32)
    t = np.array([[1, 0]], dtype=np.int32)
    a = A.paged_decode(q, kc, vc, t, [20], 1 / 8.000001, "f32")
    b = A.paged_decode(q, kc, vc, t, [20], float(np.float32(1 / 8.000001)), "f32")
    assert np.array_equal(a, b)


def test_bf16_upcast_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    vals = A.to_f64(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -1.0
    assert vals[2] == 3.140625
    assert vals[3] == 2.0 ** -133
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127


def test_out_of_pool_table_entry_is_rejected():
    q = np.ones((1, 1, 8), dtype=np.float32)
    kc = np.ones((2, 1, 16, 8), dtype=np.float32)
    vc = np.ones((2, 1, 8, 16), dtype=np.float32)
    with pytest.raises(IndexError):
        A.paged_decode(q, kc, vc, np.array([[5]], dtype=np.int32), [3], 0.3, "f32")


@pytest.mark.parametrize("pin", P.MASK_PINS, ids=[p.__name__ for p in P.MASK_PINS])
def test_mask_pin(pin):
    pin()


@pytest.mark.parametrize("pin", P.MULTI_PINS, ids=[p.__name__ for p in P.MULTI_PINS])
def test_multi_pin(pin):
    pin()


@pytest.mark.parametrize("pin", P.ROW_PINS, ids=[p.__name__ for p in P.ROW_PINS])
def test_row_pin(pin):
    pin()
