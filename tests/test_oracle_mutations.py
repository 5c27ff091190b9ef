"""Planted mistakes in the oracle (on the CPU): each must be caught by a pin.

Each case patches one piece of the oracle with a plausible error and checks
that at least one of the pins in tests/oracle_pins.py then fails.
"""
import numpy as np
import pytest

from oracle import allocator as AL
from oracle import attention as A
from oracle import cache_ops as C
from oracle import quant as Q
from tests import oracle_pins as P


def _softmax_no_shift_wrong_sign(z):
    e = np.exp(-(z - np.max(z)))
    return e / np.sum(e)


def _softmax_unnormalised(z):
    return np.exp(z - np.max(z))


def _logits_no_scale(q64, K, scale):
    return K @ q64


def _logits_sqrt_scale(q64, K, scale):
    return np.sqrt(scale) * (K @ q64)


def _gather_drop_last_row(kc, vc, row, n, g, dtype, _orig=A.gather_kv):
    K, V = _orig(kc, vc, row, n, g, dtype)
    return (K[:-1], V[:-1]) if n > 1 else (K, V)


def _gather_transposed_block(kc, vc, row, n, g, dtype, _orig=A.gather_kv):
    # reads row t of a block from the wrong KV head when there is more than one
    H_kv = kc.shape[1]
    return _orig(kc, vc, row, n, (g + 1) % H_kv, dtype)


def _merge_no_rescale(m, l, o, _orig=A.lse_merge):
    return (l @ o) / np.sum(l)


def _partials_unnormalised(q64, K, V, scale, ps, _orig=A.partition_partials):
    m, l, o = _orig(q64, K, V, scale, ps)
    return m, l, o * l[:, None]


def _per_block_softmax_decode(query, kc, vc, tables, ctx, scale, dtype):
    # one page's loop: a softmax per block, block outputs summed
    S, H, D = query.shape
    H_kv, bs = kc.shape[1], kc.shape[2]
    G = H // H_kv
    out = np.zeros((S, H, D))
    for s in range(S):
        n = int(ctx[s])
        for h in range(H):
            K, V = A.gather_kv(kc, vc, tables[s], n, h // G, dtype)
            q = A.to_f64(query[s, h], dtype)
            for j in range(0, n, bs):
                out[s, h] += A.softmax_weights(A.scale_f64(scale) * (K[j:j + bs] @ q)) @ V[j:j + bs]
    return out


ATTENTION_MUTANTS = [
    ("softmax_weights", _softmax_no_shift_wrong_sign),
    ("softmax_weights", _softmax_unnormalised),
    ("logits", _logits_no_scale),
    ("logits", _logits_sqrt_scale),
    ("gather_kv", _gather_drop_last_row),
    ("gather_kv", _gather_transposed_block),
    ("paged_decode", _per_block_softmax_decode),
]

ATTENTION_PINS = [
    lambda: P.check_against_sdpa(),
    lambda: P.check_against_sdpa(seed=5, S=2, H=8, Hkv=2, D=64, bs=16, ctx=(40, 70), dtype="f16"),
    P.check_brute_force, P.check_two_token_closed_form, P.check_identical_keys_mean,
    P.check_ctx1_is_v0, P.check_dominant_key, P.check_split_merge, P.check_p4_gather_demo,
]


def _caught(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


@pytest.mark.parametrize("name,bad", ATTENTION_MUTANTS, ids=[f"{n}:{b.__name__}" for n, b in ATTENTION_MUTANTS])
def test_attention_mutant_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(A, name, bad)
    assert _caught(ATTENTION_PINS), f"no pin caught the planted mistake in {name}"


@pytest.mark.parametrize("name,bad", [("lse_merge", _merge_no_rescale),
                                      ("partition_partials", _partials_unnormalised)])
def test_split_mutant_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(A, name, bad)
    assert _caught([P.check_split_merge])


def _kv_head_modulo(head, num_heads, num_kv_heads):
    # interleaved groups instead of contiguous ones
    return head % num_kv_heads


def _kv_head_off_by_one(head, num_heads, num_kv_heads):
    return min(num_kv_heads - 1, (head + 1) // (num_heads // num_kv_heads))


def _decode_one_group_mod(query, kc, vc, row, n, head, num_heads, scale, dtype, quant=None, mask=None):
    # the row of the right query head, but its KV head taken as head % H_kv
    g = head % kc.shape[1]
    K, V = A.kv_for(kc, vc, row, n, g, dtype, quant, mask)
    return A.attend(A.to_f64(query[head], dtype), K, V, A.scale_f64(scale))


def _decode_one_head_zero(query, kc, vc, row, n, head, num_heads, scale, dtype, quant=None, mask=None,
                          _orig=A.decode_one):
    # always the sequence's first query head
    return _orig(query, kc, vc, row, n, 0, num_heads, scale, dtype, quant, mask)


@pytest.mark.parametrize("name,bad", [("kv_head_of", _kv_head_modulo), ("kv_head_of", _kv_head_off_by_one),
                                      ("decode_one", _decode_one_group_mod),
                                      ("decode_one", _decode_one_head_zero)],
                         ids=["kv_head_of:modulo", "kv_head_of:off_by_one", "decode_one:group_mod",
                              "decode_one:head_zero"])
def test_row_mutant_is_caught(monkeypatch, name, bad):
    """A wrong head-to-group mapping, in the shared mapping or in decode_one alone, and a
    decode_one that answers for the wrong query head, each fail a pin."""
    monkeypatch.setattr(A, name, bad)
    assert _caught(ATTENTION_PINS + P.ROW_PINS), f"no pin caught the planted mistake in {name}"


class _LifoAllocator(AL.BlockAllocator):
    def _take(self):
        if not self.free:
            raise AL.AllocatorError(AL.NO_FREE_BLOCKS)
        b = self.free.pop()
        self.refs[b] = 1
        return b


class _FreeToHeadAllocator(AL.BlockAllocator):
    def _release(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.free.appendleft(b)


class _CowNoDecrement(AL.BlockAllocator):
    def seq_append_slot(self, seq_id):
        L = self.lens[seq_id]
        t = self.tables[seq_id]
        if L % self.block_size and self.refs[t[L // self.block_size]] > 1:
            self.refs[t[L // self.block_size]] += 1   # wrong: should drop by one after the copy
            self.refs[t[L // self.block_size]] -= 1
            old = t[L // self.block_size]
            new = self._take()
            t[L // self.block_size] = new
            self.lens[seq_id] = L + 1
            return new * self.block_size + L % self.block_size, old, new
        return super().seq_append_slot(seq_id)


class _CowInPlace(AL.BlockAllocator):
    def seq_append_slot(self, seq_id):
        L = self.lens[seq_id]
        if L % self.block_size:
            t = self.tables[seq_id]
            self.lens[seq_id] = L + 1
            return t[L // self.block_size] * self.block_size + L % self.block_size, -1, -1
        return super().seq_append_slot(seq_id)


class _CeilOffByOne(AL.BlockAllocator):
    def _blocks_for(self, n):
        return n // self.block_size + 1


ALLOCATOR_PINS = [P.check_p1_block_mapping, P.check_block_counts, P.check_addressing,
                  P.check_p4_cow_timeline, P.check_p2_lifecycle]


@pytest.mark.parametrize("cls", [_LifoAllocator, _FreeToHeadAllocator, _CowNoDecrement, _CowInPlace,
                                 _CeilOffByOne])
def test_allocator_mutant_is_caught(monkeypatch, cls):
    monkeypatch.setattr(AL, "BlockAllocator", cls)
    assert _caught(ALLOCATOR_PINS), f"no pin caught {cls.__name__}"


# ----------------------------------------------------------------------------
# 8-bit KV codes

def _e4m3_ties_away(y32, _orig=Q._e4m3_encode):
    import numpy as np
    out = _orig(y32)
    mag = np.abs(y32.astype(np.float64))
    pos = Q.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    at = np.isin(mag, mids)
    return np.where(at & ((out & 1) == 0) & (mag > Q.decode(out & 0x7F, "fp8_e4m3")), out + 1, out).astype(np.uint8)


def _e4m3_overflow_nan(y32, _orig=Q._e4m3_encode):
    import numpy as np
    out = _orig(y32)
    return np.where(np.abs(y32) > 448, 0x7F, out).astype(np.uint8)


def _e4m3_value_no_subnormals(code):
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0 and m:
        mag = (1.0 + m / 8.0) * 2.0 ** -7
        return -mag if code & 0x80 else mag
    return _ORIG_E4M3_VALUE(code)


_ORIG_E4M3_VALUE = Q.e4m3_value


def _quantize_multiplies(x, dtype, scale, fmt):
    import numpy as np
    return Q.encode(Q.to_f32(x, dtype) * np.float32(scale), fmt)


def _dequantize_divides(codes, scale, fmt):
    import numpy as np
    return Q.decode(codes, fmt) / float(np.float32(scale))


def _kv_swapped_scales(kc, vc, row, n, g, dtype, quant=None, mask=None, _orig=A.kv_for):
    if quant is not None:
        quant = (quant[0], quant[2], quant[1])
    return _orig(kc, vc, row, n, g, dtype, quant, mask)


def _int8_ties_away(y32):
    import numpy as np
    y = y32.astype(np.float64)
    r = np.clip(np.sign(y) * np.floor(np.abs(np.nan_to_num(y)) + 0.5), -127, 127)
    return r.astype(np.int64).astype(np.uint8)


def _int8_asymmetric(y32):
    import numpy as np
    y = np.nan_to_num(y32.astype(np.float64))
    return np.clip(np.rint(y), -128, 127).astype(np.int64).astype(np.uint8)


QUANT_MUTANTS = [
    (Q, "_e4m3_encode", _e4m3_ties_away),
    (Q, "_e4m3_encode", _e4m3_overflow_nan),
    (Q, "quantize", _quantize_multiplies),
    (Q, "dequantize", _dequantize_divides),
    (A, "kv_for", _kv_swapped_scales),
    (Q, "_int8_encode", _int8_ties_away),
    (Q, "_int8_encode", _int8_asymmetric),
]


@pytest.mark.parametrize("mod,name,bad", QUANT_MUTANTS, ids=[f"{n}:{b.__name__}" for _, n, b in QUANT_MUTANTS])
def test_quant_mutant_is_caught(monkeypatch, mod, name, bad):
    monkeypatch.setattr(mod, name, bad)
    assert _caught(P.QUANT_PINS), f"no pin caught the planted mistake in {name}"


def _rows_mean_scale(x, dtype, _orig=Q.quantize_rows_int8):
    # scale from the mean magnitude instead of the largest
    import numpy as np
    x32 = Q.to_f32(x, dtype)
    sc = (np.mean(np.abs(x32), axis=-1) / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        codes = Q.encode(x32 / sc[..., None], "int8")
    return codes, sc


def _rows_scale_255(x, dtype):
    # the full byte range instead of the symmetric 127
    import numpy as np
    x32 = Q.to_f32(x, dtype)
    sc = (np.max(np.abs(x32), axis=-1) / np.float32(255)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        codes = Q.encode(x32 / sc[..., None], "int8")
    return codes, sc


def _rows_dequant_ignores_scale(codes, scales):
    return Q.decode(codes, "int8") * 0.01


def _row_scales_of_next_head(scale_pool, table_row, positions, kv_head, _orig=A.gather_row_scales):
    return _orig(scale_pool, table_row, positions, (kv_head + 1) % scale_pool.shape[1])


def _token_write_keeps_old_scales(key, value, kc, vc, ks, vs, slots, dtype, _orig=C.reshape_and_cache_int8_token):
    kc2, vc2, _, _ = _orig(key, value, kc, vc, ks, vs, slots, dtype)
    return kc2, vc2, ks.copy(), vs.copy()


TOKEN_MUTANTS = [
    (Q, "quantize_rows_int8", _rows_mean_scale),
    (Q, "quantize_rows_int8", _rows_scale_255),
    (Q, "dequantize_rows_int8", _rows_dequant_ignores_scale),
    (A, "gather_row_scales", _row_scales_of_next_head),
    (C, "reshape_and_cache_int8_token", _token_write_keeps_old_scales),
]


@pytest.mark.parametrize("mod,name,bad", TOKEN_MUTANTS, ids=[f"{n}:{b.__name__}" for _, n, b in TOKEN_MUTANTS])
def test_token_scale_mutant_is_caught(monkeypatch, mod, name, bad):
    """Planted mistakes in the per-(token, KV head) int8 form: each fails a pin."""
    monkeypatch.setattr(mod, name, bad)
    assert _caught(P.TOKEN_PINS), f"no pin caught the planted mistake in {name}"


def test_quant_table_mutant_is_caught(monkeypatch):
    import numpy as np
    table = np.array([_e4m3_value_no_subnormals(c) for c in range(256)])
    monkeypatch.setattr(Q, "E4M3_TABLE", table)
    monkeypatch.setattr(Q, "_POS_VALUES", table[:0x7F])
    assert _caught(P.QUANT_PINS)


# ----------------------------------------------------------------------------
# prefix caching

class _PrefixAlwaysMiss(AL.BlockAllocator):
    def prefix_get_or_create(self, tokens):
        self.prefixes.pop(tuple(int(t) for t in tokens), None)   # forgets every entry
        return super().prefix_get_or_create(tokens)


class _PrefixNoHole(AL.BlockAllocator):
    def seq_create_with_prefix(self, seq_id, pid, own_tokens):
        # own tokens continue right after the prefix, in the prefix's last block
        e = self._entry(pid)
        n = e["length"] + own_tokens
        for b in e["blocks"]:
            self.refs[b] += 1
        extra = self._blocks_for(n) - len(e["blocks"])
        self.tables[seq_id] = list(e["blocks"]) + [self._take() for _ in range(max(extra, 0))]
        self.lens[seq_id] = n


class _PrefixReleaseKeepsBlocks(AL.BlockAllocator):
    def prefix_release(self, pid):
        e = self._entry(pid)
        e["users"] -= 1
        if e["users"] <= 0:
            del self.prefixes[e["key"]]
            del self.entries[pid]


@pytest.mark.parametrize("cls", [_PrefixAlwaysMiss, _PrefixNoHole, _PrefixReleaseKeepsBlocks])
def test_prefix_mutant_is_caught(monkeypatch, cls):
    monkeypatch.setattr(AL, "BlockAllocator", cls)
    assert _caught([P.check_p4_prefix_demo]), f"no pin caught {cls.__name__}"


# ----------------------------------------------------------------------------
# masked positions

def _keep_off_by_one(num_tokens, lo, hi):
    import numpy as np
    t = np.arange(num_tokens)
    return t[(t < lo) | (t > hi)]


def _keep_ignores_mask(num_tokens, lo, hi):
    import numpy as np
    return np.arange(num_tokens)


def _merge_unguarded(m, l, o):
    import numpy as np
    if m.shape[0] == 0:
        return np.zeros(o.shape[1])
    M = np.max(m)
    w = l * np.exp(m - M)
    return (w @ o) / np.sum(w)


@pytest.mark.parametrize("name,bad", [("keep_positions", _keep_off_by_one), ("keep_positions", _keep_ignores_mask),
                                      ("lse_merge", _merge_unguarded)])
def test_mask_mutant_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(A, name, bad)
    assert _caught(P.MASK_PINS), f"no pin caught {bad.__name__}"


# ----------------------------------------------------------------------------
# several query tokens per sequence

def _multi_not_causal(query, kc, vc, tables, ctx, qstart, scale, dtype, quant=None):
    import numpy as np
    T, H, D = query.shape
    out = np.zeros((T, H, D))
    for s in range(len(ctx)):
        for r in range(int(qstart[s]), int(qstart[s + 1])):
            out[r] = A.paged_decode(query[r:r + 1], kc, vc, tables[s:s + 1], [ctx[s]], scale, dtype, quant)[0]
    return out


def _multi_off_by_one(query, kc, vc, tables, ctx, qstart, scale, dtype, quant=None):
    import numpy as np
    T, H, D = query.shape
    out = np.zeros((T, H, D))
    for s in range(len(ctx)):
        n, L = int(ctx[s]), int(qstart[s + 1] - qstart[s])
        for i in range(L):
            lim = max(1, n - L + i)      # forgets that the token sees itself
            r = int(qstart[s]) + i
            out[r] = A.paged_decode(query[r:r + 1], kc, vc, tables[s:s + 1], [lim], scale, dtype, quant)[0]
    return out


@pytest.mark.parametrize("bad", [_multi_not_causal, _multi_off_by_one])
def test_multi_mutant_is_caught(monkeypatch, bad):
    monkeypatch.setattr(A, "paged_decode_multi", bad)
    assert _caught(P.MULTI_PINS), f"no pin caught {bad.__name__}"


# ----------------------------------------------------------------------------
# swap and sliding window

class _SwapOutKeepsDeviceRefs(AL.BlockAllocator):
    def _release(self, b):
        if self.swapped is not None and getattr(self, "_in_swap", False):
            return
        super()._release(b)

    def seq_swap_out(self, seq_ids):
        self._in_swap = True
        try:
            return super().seq_swap_out(seq_ids)
        finally:
            self._in_swap = False


class _SwapInUnshares(AL.BlockAllocator):
    def seq_swap_in(self, seq_ids):
        pairs = super().seq_swap_in(seq_ids)
        # gives every reference its own device copy (loses sharing inside the group)
        seen = set()
        for s in seq_ids:
            t = self.tables[s]
            for j, b in enumerate(t):
                if b in seen and b >= 0:
                    self.refs[b] -= 1
                    n = self._take()
                    t[j] = n
                    pairs.append((-1, n))
                seen.add(b)
        return pairs


class _WindowOffByOneBlock(AL.BlockAllocator):
    def _drop_behind_window(self, seq_id):
        start = self.lens[seq_id] - self.windows[seq_id] + self.block_size
        t = self.tables[seq_id]
        for j in range(len(t)):
            if (j + 1) * self.block_size > start:
                break
            if t[j] >= 0:
                self._release(t[j])
                t[j] = -1


@pytest.mark.parametrize("cls", [_SwapOutKeepsDeviceRefs, _SwapInUnshares, _WindowOffByOneBlock])
def test_swap_window_mutant_is_caught(monkeypatch, cls):
    monkeypatch.setattr(AL, "BlockAllocator", cls)
    assert _caught(P.SWAP_WINDOW_PINS), f"no pin caught {cls.__name__}"
