"""Checks that pin the CPU oracle to things other than itself.

Each check raises AssertionError when the oracle is wrong.  They are used
twice: by the CPU tests on the real oracle, and by tests/test_oracle_mutations.py
on copies of the oracle with a planted mistake, to show each pin has teeth.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import attention as A
from oracle import allocator as AL
from oracle import cache_ops as C
from synth import normal_host

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def ceil_div(a, b):
    return -(-a // b)


def scatter_case(seed, S, H, Hkv, D, bs, ctx, dtype, extra_blocks=3):
    """Contiguous per-sequence K/V, scattered into a pool through random tables.

    Returns (query, key_cache, value_cache, tables, ctx, contiguous K list, V list);
    the contiguous lists are float64 [Hkv, n, D] built independently of the oracle's
    gather, so a gather mistake cannot hide.
    """
    rng = np.random.default_rng(seed)
    need = [ceil_div(n, bs) for n in ctx]
    NB = sum(need) + extra_blocks
    MB = max(need + [1])
    perm = rng.permutation(NB)
    tables = -np.ones((S, MB), dtype=np.int32)
    pos = 0
    for s in range(S):
        tables[s, : need[s]] = perm[pos:pos + need[s]]
        pos += need[s]
    kc = normal_host((NB, Hkv, bs, D), seed + 1, dtype)
    vc = normal_host((NB, Hkv, D, bs), seed + 2, dtype)
    q = normal_host((S, H, D), seed + 3, dtype)
    Ks, Vs = [], []
    for s in range(S):
        n = ctx[s]
        K = np.zeros((Hkv, n, D))
        V = np.zeros((Hkv, n, D))
        for t in range(n):
            b = tables[s, t // bs]
            K[:, t] = A.to_f64(kc[b, :, t % bs], dtype)
            V[:, t] = A.to_f64(vc[b, :, :, t % bs], dtype)
        Ks.append(K)
        Vs.append(V)
    return q, kc, vc, tables, list(ctx), Ks, Vs


def check_against_sdpa(seed=7, S=3, H=8, Hkv=2, D=64, bs=16, ctx=(1, 37, 80), dtype="f32"):
    """The paged oracle equals torch's float64 scaled-dot-product attention run on the
    contiguous cache (an independent library implementation of the textbook formula;
    grouped heads via its enable_gqa, which groups query heads contiguously)."""
    import torch
    import torch.nn.functional as F

    q, kc, vc, tables, ctx, Ks, Vs = scatter_case(seed, S, H, Hkv, D, bs, ctx, dtype)
    scale = 1.0 / math.sqrt(D)
    out = A.paged_decode(q, kc, vc, tables, ctx, scale, dtype)
    for s in range(S):
        qt = torch.from_numpy(A.to_f64(q[s], dtype)).view(1, H, 1, D)
        kt = torch.from_numpy(Ks[s]).view(1, Hkv, ctx[s], D)
        vt = torch.from_numpy(Vs[s]).view(1, Hkv, ctx[s], D)
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=float(np.float32(scale)),
                                             enable_gqa=(H != Hkv)).view(H, D).numpy()
        assert np.max(np.abs(out[s] - ref)) <= 1e-12, f"seq {s}: oracle differs from SDPA"


def check_brute_force(seed=11, n=23, D=16):
    """Softmax written without the max shift, summed with math.fsum, on tiny inputs."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    V = rng.standard_normal((n, D))
    scale = 0.25
    z = [scale * math.fsum(q[d] * K[t, d] for d in range(D)) for t in range(n)]
    den = math.fsum(math.exp(x) for x in z)
    ref = np.array([math.fsum(math.exp(z[t]) * V[t, d] for t in range(n)) / den for d in range(D)])
    out = A.attend(q, K, V, scale)
    assert np.max(np.abs(out - ref)) <= 1e-12


def check_two_token_closed_form(seed=5, D=32):
    """n = 2: the weights are logistic functions of the logit difference."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(D)
    K = rng.standard_normal((2, D))
    V = rng.standard_normal((2, D))
    scale = 1 / math.sqrt(D)
    d = scale * (float(np.dot(q, K[0])) - float(np.dot(q, K[1])))
    w0 = 1.0 / (1.0 + math.exp(-d))
    ref = w0 * V[0] + (1.0 - w0) * V[1]
    assert np.max(np.abs(A.attend(q, K, V, scale) - ref)) <= 1e-13


def check_identical_keys_mean(seed=3, n=45, D=64):
    """All keys equal -> uniform weights -> the plain mean of V."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(D)
    K = np.tile(rng.standard_normal(D), (n, 1))
    V = rng.standard_normal((n, D))
    out = A.attend(q, K, V, 0.125)
    assert np.max(np.abs(out - V.mean(axis=0))) <= 1e-14 * max(1.0, np.max(np.abs(V)))


def check_ctx1_is_v0(seed=9, D=64):
    rng = np.random.default_rng(seed)
    q, K, V = rng.standard_normal(D), rng.standard_normal((1, D)), rng.standard_normal((1, D))
    assert np.array_equal(A.attend(q, K, V, 0.125), V[0])


def check_dominant_key(seed=13, n=30, D=64):
    """One key aligned with q and far larger in its logit takes all the weight."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D)) * 0.01
    j = 17
    K[j] = q * (400.0 / np.dot(q, q))  # logit 400 * scale vs ~0 for the others
    V = rng.standard_normal((n, D))
    out = A.attend(q, K, V, 0.5)
    assert np.max(np.abs(out - V[j])) <= 1e-12


def check_permutation_invariance(seed=21, dtype="f16"):
    """Relabelling physical blocks (pool'[pi(b)] = pool[b], table' = pi(table)) changes nothing."""
    q, kc, vc, tables, ctx, _, _ = scatter_case(seed, 3, 4, 4, 64, 16, (5, 33, 64), dtype)
    NB = kc.shape[0]
    rng = np.random.default_rng(seed + 100)
    pi = rng.permutation(NB)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    a = A.paged_decode(q, kc, vc, tables, ctx, 0.125, dtype)
    b = A.paged_decode(q, kc2, vc2, t2, ctx, 0.125, dtype)
    assert np.array_equal(a, b)


def check_key_shift_invariance(seed=17, n=40, D=32):
    """Adding one vector w to every key shifts all logits equally: output unchanged."""
    rng = np.random.default_rng(seed)
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    w = rng.standard_normal(D) * 3
    a = A.attend(q, K, V, 0.3)
    b = A.attend(q, K + w, V, 0.3)
    assert np.max(np.abs(a - b)) <= 1e-12


def check_value_affine(seed=19, n=40, D=32):
    """Weights sum to one: out(aV + b) = a out(V) + b."""
    rng = np.random.default_rng(seed)
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    bvec = rng.standard_normal(D)
    a = A.attend(q, K, V, 0.3)
    b = A.attend(q, K, 2.5 * V + bvec, 0.3)
    assert np.max(np.abs(b - (2.5 * a + bvec))) <= 1e-12


def check_split_merge(seed=23, n=1300, D=32):
    """Partials over any partition size merge back to the direct result; with one token per
    partition the partials are (z_t, 1, V_t) and the merge is the softmax itself."""
    rng = np.random.default_rng(seed)
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    scale = 1 / math.sqrt(D)
    direct = A.attend(q, K, V, scale)
    for ps in (1, 7, 16, 512, n, n + 5):
        m, l, o = A.partition_partials(q, K, V, scale, ps)
        assert m.shape[0] == ceil_div(n, ps)
        assert np.max(np.abs(A.lse_merge(m, l, o) - direct)) <= 1e-12, f"partition {ps}"
    m, l, o = A.partition_partials(q, K[:9], V[:9], scale, 1)
    assert np.allclose(m, scale * (K[:9] @ q), rtol=0, atol=1e-15)
    assert np.array_equal(l, np.ones(9))
    assert np.array_equal(o, V[:9])
    # the merge alone, on hand-made partials whose answer is known in closed form
    mm = np.array([0.0, math.log(3.0)])
    ll = np.array([1.0, 1.0])
    oo = np.array([[1.0, 0.0], [0.0, 1.0]])
    assert np.max(np.abs(A.lse_merge(mm, ll, oo) - np.array([0.25, 0.75]))) <= 1e-15


def check_kv_head_mapping():
    """Contiguous groups: with 32 query heads on 8 KV heads, heads 4k..4k+3 read KV head k;
    MHA maps each head to itself and one KV head serves every query head."""
    assert [A.kv_head_of(h, 32, 8) for h in range(32)] == [h // 4 for h in range(32)]
    assert [A.kv_head_of(h, 6, 2) for h in range(6)] == [0, 0, 0, 1, 1, 1]
    assert [A.kv_head_of(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    assert [A.kv_head_of(h, 8, 1) for h in range(8)] == [0] * 8
    for bad in ((0, 6, 4), (6, 6, 2), (-1, 4, 4)):
        try:
            A.kv_head_of(*bad)
        except (ValueError, IndexError):
            continue
        raise AssertionError(f"kv_head_of accepted {bad}")


def check_decode_one_rows(seed=29):
    """decode_one gives row (s, h) of paged_decode bit for bit, for every query head of GQA
    and MHA shapes on permuted tables: with the full pools and the sequence's whole query,
    and with the pools cut to the one KV head that head reads (as a caller that fetched only
    those blocks passes them).  Each row also equals torch's float64 SDPA on the contiguous
    cache, so a wrong head or group index cannot agree with paged_decode by accident."""
    import torch
    import torch.nn.functional as F

    for S, H, Hkv, D, bs, ctx, dtype in ((3, 8, 2, 32, 16, (1, 37, 80), "f32"),
                                          (2, 32, 8, 64, 32, (45, 130), "bf16"),
                                          (2, 6, 3, 32, 16, (17, 64), "f16"),
                                          (2, 4, 4, 32, 16, (20, 33), "f16")):
        q, kc, vc, tables, ctx, Ks, Vs = scatter_case(seed + H, S, H, Hkv, D, bs, ctx, dtype)
        scale = 1.0 / math.sqrt(D)
        full = A.paged_decode(q, kc, vc, tables, ctx, scale, dtype)
        G = H // Hkv
        for s in range(S):
            qt = torch.from_numpy(A.to_f64(q[s], dtype)).view(1, H, 1, D)
            kt = torch.from_numpy(Ks[s]).view(1, Hkv, ctx[s], D)
            vt = torch.from_numpy(Vs[s]).view(1, Hkv, ctx[s], D)
            sdpa = F.scaled_dot_product_attention(qt, kt, vt, scale=float(np.float32(scale)),
                                                  enable_gqa=(H != Hkv)).view(H, D).numpy()
            for h in range(H):
                row = A.decode_one(q[s], kc, vc, tables[s], ctx[s], h, H, scale, dtype)
                assert np.array_equal(row, full[s, h]), f"{(S, H, Hkv)} seq {s} head {h}: differs from paged_decode"
                assert np.max(np.abs(row - sdpa[h])) <= 1e-12, f"{(S, H, Hkv)} seq {s} head {h}: differs from SDPA"
                g = h // G
                cut = A.decode_one(q[s], kc[:, g:g + 1], vc[:, g:g + 1], tables[s], ctx[s], h, H, scale, dtype)
                assert np.array_equal(cut, row), f"seq {s} head {h}: the one-KV-head form differs"


def check_decode_one_masked_and_8bit(seed=31):
    """decode_one with a mask, and over 8-bit pools, gives paged_decode's row (both pinned
    on their own: the masked form against SDPA, the 8-bit form against float pools)."""
    from oracle import quant as Q
    S, H, Hkv, D, bs = 3, 8, 2, 32, 16
    q, kc, vc, tables, ctx, _, _ = scatter_case(seed, S, H, Hkv, D, bs, (46, 90, 33), "f16")
    lo, hi = [9, 0, 5], [16, 66, 5]
    ref = A.paged_decode(q, kc, vc, tables, ctx, 0.2, "f16", masks=(lo, hi))
    for s in range(S):
        for h in range(H):
            row = A.decode_one(q[s], kc, vc, tables[s], ctx[s], h, H, 0.2, "f16", mask=(lo[s], hi[s]))
            assert np.array_equal(row, ref[s, h]), f"masked seq {s} head {h}"
    NB = kc.shape[0]
    for fmt in Q.FORMATS:
        k8, v8 = _lossless_pools(fmt, seed + 5, NB, Hkv, bs, D)
        quant = (fmt, 0.125, 0.5)
        ref = A.paged_decode(q, k8, v8, tables, ctx, 0.2, "f16", quant=quant)
        for s in range(S):
            for h in range(H):
                row = A.decode_one(q[s], k8, v8, tables[s], ctx[s], h, H, 0.2, "f16", quant=quant)
                assert np.array_equal(row, ref[s, h]), f"{fmt} seq {s} head {h}"


ROW_PINS = [check_kv_head_mapping, check_decode_one_rows, check_decode_one_masked_and_8bit]


def check_p4_gather_demo():
    """Table [3, 7, 12, 21] with 50 valid tokens: 4 blocks, the last holds 2 rows (12% full)."""
    g = golden("block_counts.json")
    case = [c for c in g["cases"] if c["source"] == "impl"][0]
    bs, n, table = case["block_size"], case["tokens"], case["table"]
    kc = normal_host((24, 1, bs, 8), 5, "f32")
    vc = normal_host((24, 1, 8, bs), 6, "f32")
    K, V = A.gather_kv(kc, vc, np.array(table), n, 0, "f32")
    assert K.shape == (n, 8)
    assert A.blocks_for(n, bs) == case["blocks"] == len(table)
    rows_last = n - (case["blocks"] - 1) * bs
    assert rows_last == case["last_block_rows"]
    assert f"{(n % bs) / bs * 100:.0f}%" == case["last_block_fill_printed"]
    assert np.array_equal(K[48:50], kc[21, 0, 0:2].astype(np.float64))
    assert np.array_equal(V[16:32], vc[7, 0].T.astype(np.float64))


# --------------------------------------------------------------------------- allocator


def check_p1_block_mapping():
    g = golden("p1_block_mapping.json")
    al = AL.BlockAllocator(g["num_blocks"], g["block_size"])
    for rid, tokens in g["requests"]:
        al.seq_create(rid, tokens)
    for rid, table in g["expected_tables"].items():
        assert al.block_table(int(rid)) == table
    used = sorted(b for rid in g["expected_tables"] for b in al.block_table(int(rid)))
    assert used == g["expected_used"]
    assert al.free_list()[:3] == g["expected_free_head"]
    al.seq_free(g["free_request"])
    assert al.free_list()[-2:] == g["expected_free_tail_after_free"]


def check_block_counts():
    g = golden("block_counts.json")
    for c in g["cases"]:
        al = AL.BlockAllocator(16, c["block_size"])
        al.seq_create(1, c["tokens"])
        assert len(al.block_table(1)) == c["blocks"]
        if "slots" in c:
            assert len(al.block_table(1)) * c["block_size"] == c["slots"]


def check_addressing():
    g = golden("addressing.json")
    bs = g["block_size"]
    al = AL.BlockAllocator(12, bs, initial_free_order=[3, 7, 11] + [b for b in range(12) if b not in (3, 7, 11)])
    al.seq_create(1, 0)
    slots = []
    for t in range(max(g["tokens"]) + 1):
        slot, src, dst = al.seq_append_slot(1)
        assert src == dst == -1
        slots.append(slot)
    assert al.block_table(1) == g["table"]
    assert [slots[t] for t in g["tokens"]] == g["expected_slot"]
    assert [slots[t] // bs for t in g["tokens"]] == [g["table"][lb] for lb in g["expected_logical_block"]]
    assert [slots[t] % bs for t in g["tokens"]] == g["expected_offset"]


def check_p4_cow_timeline():
    g = golden("p4_cow_timeline.json")
    nb, bs = g["num_blocks"], g["block_size"]
    head = g["free_order_head"]
    order = head + [b for b in range(nb) if b not in head]
    al = AL.BlockAllocator(nb, bs, order)
    al.seq_create("A", g["seq_a_tokens"])
    al.seq_fork("A", "B")
    assert al.ref_count(5) == g["expected_before"]["ref_5"]
    slot, src, dst = al.seq_append_slot("B")
    ea = g["expected_after"]
    assert [src, dst] == ea["cow_pair"]
    assert slot == ea["slot_b"]
    assert al.ref_count(5) == ea["ref_5"] and al.ref_count(42) == ea["ref_42"]
    assert al.block_table("A") == ea["table_a"] and al.block_table("B") == ea["table_b"]
    # data: copy then write; the two blocks differ only at the written offset
    kc = normal_host((nb, 2, bs, 4), 1, "f16")
    vc = normal_host((nb, 2, 4, bs), 2, "f16")
    kc, vc = C.copy_blocks(kc, vc, [[src, dst]])
    newk = normal_host((1, 2, 4), 3, "f16")
    newv = normal_host((1, 2, 4), 4, "f16")
    kc, vc = C.reshape_and_cache(newk, newv, kc, vc, [slot])
    differ = [o for o in range(bs) if not np.array_equal(kc[5, :, o], kc[42, :, o])]
    assert differ == [ea["differs_only_at_offset"]]
    differ_v = [o for o in range(bs) if not np.array_equal(vc[5, :, :, o], vc[42, :, :, o])]
    assert differ_v == [ea["differs_only_at_offset"]]
    assert np.array_equal(kc[42, :, 8], newk[0]) and np.array_equal(vc[42, :, :, 8], newv[0])


def check_p2_lifecycle():
    g = golden("p2_refcount_lifecycle.json")
    al = AL.BlockAllocator(g["num_blocks"], g["block_size"])
    first = None
    for st in g["steps"]:
        if st["op"] == "create":
            al.seq_create(st["seq"], st["tokens"])
            first = al.block_table(st["seq"])[0]
        elif st["op"] == "fork":
            al.seq_fork(st["parent"], st["child"])
        elif st["op"] == "free":
            al.seq_free(st["seq"])
        assert al.ref_count(first) == st["expect_ref0"]
        assert al.num_free_blocks() == st["expect_free"]


# ----------------------------------------------------------------------------
# 8-bit KV codes (oracle/quant.py)

def check_e4m3_special_values():
    """Fixed points of the OCP FP8 E4M3 ("fn") format: bias 7, three mantissa
    bits, subnormals below 2^-6, no infinities, NaN only at S.1111.111."""
    from oracle import quant as Q
    t = Q.E4M3_TABLE
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0
    assert t[0x3C] == 1.5
    assert t[0x7E] == 448.0              # largest finite
    assert t[0xFE] == -448.0
    nan = [c for c in range(256) if np.isnan(t[c])]
    assert nan == [0x7F, 0xFF], nan
    assert not np.isinf(t).any()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must increase"
    assert np.array_equal(t[0x80:0xFF], -pos)


def check_e4m3_table_vs_torch():
    """The code table against torch's float8_e4m3fn (an independent decoder)."""
    import torch
    from oracle import quant as Q
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ref == Q.E4M3_TABLE) | (np.isnan(ref) & np.isnan(Q.E4M3_TABLE))
    assert same.all(), np.nonzero(~same)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(Q.E4M3_TABLE[fin]))


def _e4m3_probe_values(seed):
    from oracle import quant as Q
    rng = np.random.default_rng(seed)
    pos = Q.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2            # every tie between neighbours
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    mags = np.exp2(rng.uniform(-12, 9, size=4000))
    mags = mags[mags <= 464]
    y = np.concatenate([pos, mids, near.astype(np.float64), mags, [464.0, 2.0 ** -10, 2.0 ** -11]])
    y = y.astype(np.float32)
    sign = np.where(rng.random(y.shape) < 0.5, -1, 1).astype(np.float32)
    return np.concatenate([y, y * sign])


def check_e4m3_encode_vs_torch(seed=31):
    """Encoding agrees with torch's round-to-nearest-even cast wherever that
    cast does not overflow (|y| <= 464), ties and subnormals included."""
    import torch
    from oracle import quant as Q
    y = _e4m3_probe_values(seed)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = Q.encode(y, "fp8_e4m3")
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(y[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


def check_e4m3_round_trip():
    from oracle import quant as Q
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = Q.decode(codes, "fp8_e4m3").astype(np.float32)
    assert np.array_equal(Q.encode(vals, "fp8_e4m3"), codes)


def check_e4m3_saturation():
    """Saturation past +-448 and the NaN code (the chosen readings)."""
    from oracle import quant as Q
    y = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e30, np.inf, -449.0, -np.inf, np.nan],
                 dtype=np.float32)
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F]
    assert Q.encode(y, "fp8_e4m3").tolist() == want


def check_int8_encode(seed=37):
    """int8 codes: nearest integer by brute force over [-127, 127], ties to
    the even integer, against torch.round; saturation; NaN -> 0."""
    import torch
    from oracle import quant as Q
    rng = np.random.default_rng(seed)
    y = np.concatenate([rng.uniform(-140, 140, size=3000), np.arange(-130, 131) + 0.5,
                        [-0.5, 0.5, 1.5, 2.5, -2.5]]).astype(np.float32)
    got = Q.encode(y, "int8").view(np.int8).astype(np.int64)
    ks = np.arange(-127, 128)
    d = np.abs(y.astype(np.float64)[:, None] - ks[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = (d == best)
    brute = np.where((cand & (ks % 2 == 0)).any(axis=1), ks[np.argmax(cand & (ks % 2 == 0), axis=1)],
                     ks[np.argmax(cand, axis=1)])
    assert np.array_equal(got, brute)
    ref = torch.clamp(torch.round(torch.from_numpy(y)), -127, 127).to(torch.int64).numpy()
    assert np.array_equal(got, ref)
    special = Q.encode(np.array([np.inf, -np.inf, np.nan, 1e9, -1e9], np.float32), "int8").view(np.int8)
    assert special.tolist() == [127, -127, 0, 127, -127]
    assert Q.INT8_TABLE[0x80] == -128 and Q.INT8_TABLE[0xFF] == -1 and Q.INT8_TABLE[0x7F] == 127


def check_quantize_division(seed=41):
    """quantize(x, scale) takes the code of the float32 quotient x / scale:
    compared with torch computing the quotient and casting on its own."""
    import torch
    from oracle import quant as Q
    x = normal_host((4000,), seed, "f16")
    for scale in (5.0 / 448, 0.3, 1.0 / 7):
        tq = torch.from_numpy(x.astype(np.float32)) / torch.tensor(scale, dtype=torch.float32)
        ref8 = tq.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(Q.quantize(x, "f16", scale, "fp8_e4m3"), ref8)
        refi = torch.clamp(torch.round(tq * 100), -127, 127)  # a wider spread for int8
        xi = (x.astype(np.float32) * np.float32(100)).astype(np.float16)
        tqi = torch.from_numpy(xi.astype(np.float32)) / torch.tensor(scale, dtype=torch.float32)
        refi = torch.clamp(torch.round(tqi), -127, 127).to(torch.int8).view(torch.uint8).numpy()
        assert np.array_equal(Q.quantize(xi, "f16", scale, "int8"), refi)


def _lossless_pools(fmt, seed, NB, Hkv, bs, D):
    """Random non-NaN codes and the float32 values they stand for at scale 1."""
    from oracle import quant as Q
    rng = np.random.default_rng(seed)
    allowed = np.array([c for c in range(256) if not np.isnan(Q.decode(c, fmt))], dtype=np.uint8)
    allowed = allowed[np.abs(Q.decode(allowed, fmt)) <= 8]  # keeps the logits moderate
    kc8 = rng.choice(allowed, size=(NB, Hkv, bs, D))
    vc8 = rng.choice(allowed, size=(NB, Hkv, D, bs))
    return kc8, vc8


def check_quant_attention_lossless(seed=43):
    """Pools whose values are exactly code * scale (power-of-two scales, K and
    V different): attention over the 8-bit pools equals attention over the
    same values stored in float32."""
    from oracle import quant as Q
    S, H, Hkv, D, bs = 3, 8, 2, 32, 16
    ctx = [1, 29, 64]
    NB = 16
    k_scale, v_scale = 0.125, 4.0
    rng = np.random.default_rng(seed)
    tables = np.stack([rng.permutation(NB)[:4] for _ in range(S)]).astype(np.int32)
    q = normal_host((S, H, D), seed + 1, "f32")
    for fmt in Q.FORMATS:
        kc8, vc8 = _lossless_pools(fmt, seed + 2, NB, Hkv, bs, D)
        kf = (Q.decode(kc8, fmt) * k_scale).astype(np.float32)
        vf = (Q.decode(vc8, fmt) * v_scale).astype(np.float32)
        want = A.paged_decode(q, kf, vf, tables, ctx, 0.25, "f32")
        got = A.paged_decode(q, kc8, vc8, tables, ctx, 0.25, "f32", quant=(fmt, k_scale, v_scale))
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want))), fmt


def check_quant_write_round_trip(seed=47):
    """Rows made of code * scale values, written through the quantising
    slot-mapping write, read back as exactly those values."""
    from oracle import quant as Q
    NB, Hkv, bs, D = 6, 2, 16, 32
    k_scale, v_scale = 0.0625, 2.0
    rng = np.random.default_rng(seed)
    for fmt in Q.FORMATS:
        kc8, vc8 = _lossless_pools(fmt, seed, NB, Hkv, bs, D)
        n = 9
        slots = rng.choice(NB * bs, size=n, replace=False).astype(np.int32)
        kcode, vcode = _lossless_pools(fmt, seed + 1, n, Hkv, 1, D)
        kv = (Q.decode(kcode[:, :, 0, :], fmt) * k_scale).astype(np.float32)
        vv = (Q.decode(vcode[:, :, :, 0], fmt) * v_scale).astype(np.float32)
        kc2, vc2 = C.reshape_and_cache_quant(kv, vv, kc8, vc8, slots, "f32", fmt, k_scale, v_scale)
        for i, slot in enumerate(slots.tolist()):
            b, o = divmod(slot, bs)
            assert np.array_equal(Q.dequantize(kc2[b, :, o, :], k_scale, fmt), kv[i].astype(np.float64))
            assert np.array_equal(Q.dequantize(vc2[b, :, :, o], v_scale, fmt), vv[i].astype(np.float64))
        untouched = np.ones((NB, bs), bool)
        for slot in slots.tolist():
            untouched[slot // bs, slot % bs] = False
        assert np.array_equal(kc2.transpose(0, 2, 1, 3)[untouched], kc8.transpose(0, 2, 1, 3)[untouched])


QUANT_PINS = [check_e4m3_special_values, check_e4m3_table_vs_torch, check_e4m3_encode_vs_torch,
              check_e4m3_round_trip, check_e4m3_saturation, check_int8_encode, check_quantize_division,
              check_quant_attention_lossless, check_quant_write_round_trip]

# ----------------------------------------------------------------------------
# int8 with one scale per (token, KV head)

def check_int8_rows_closed_forms(seed=51):
    """Per-row int8 codes: the largest |element| of a row maps to +-127 with its sign, every
    element is within half a code step (s / 2) of code * s, a row of zeros has scale 0 and
    codes 0, and a row of whole multiples of 2^k whose largest is 127 * 2^k comes back exactly."""
    from oracle import quant as Q
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((40, 64)) * rng.uniform(0.01, 50, size=(40, 1))).astype(np.float32)
    codes, sc = Q.quantize_rows_int8(x, "f32")
    vals = Q.decode(codes, "int8")
    for r in range(x.shape[0]):
        j = int(np.argmax(np.abs(x[r])))
        assert vals[r, j] == (127.0 if x[r, j] > 0 else -127.0), r
        assert np.max(np.abs(x[r] - vals[r] * float(sc[r]))) <= 0.50001 * float(sc[r]), r
        assert np.max(np.abs(vals[r])) == 127.0
    c0, s0 = Q.quantize_rows_int8(np.zeros((3, 8), np.float32), "f32")
    assert not c0.any() and not s0.any()
    k = np.array([-7, -3, 0, 2, 5], dtype=np.float64)
    row = np.concatenate([rng.integers(-126, 127, size=30), [127]]).astype(np.float64)
    for e in k:
        xs = (row * 2.0 ** e).astype(np.float32)[None, :]
        c, s_ = Q.quantize_rows_int8(xs, "f32")
        assert float(s_[0]) == 2.0 ** e
        assert np.array_equal(Q.dequantize_rows_int8(c, s_), xs.astype(np.float64))
    # bf16 and fp16 inputs are widened exactly first
    xb = np.array([[0x3F80, 0xC000, 0x3E80]], dtype=np.uint16)   # 1, -2, 0.25
    cb, sb = Q.quantize_rows_int8(xb, "bf16")
    assert float(sb[0]) == float(np.float32(2.0) / np.float32(127)) and Q.decode(cb, "int8")[0, 1] == -127.0


def check_int8_rows_vs_torch(seed=53):
    """Per-row int8 codes and scales equal torch's float32 amax / 127 and round-half-even of
    the quotient, clamped to +-127, on normal rows, rows with ties and fp16 rows."""
    import torch
    from oracle import quant as Q
    rng = np.random.default_rng(seed)
    rows = [rng.standard_normal((50, 128)).astype(np.float32)]
    tie = np.zeros((4, 16), np.float32)
    tie[:, 0] = 127.0
    tie[:, 1:] = np.arange(15, dtype=np.float32) + 0.5        # quotients k + 0.5 exactly
    rows.append(tie)
    rows.append(rng.standard_normal((20, 64)).astype(np.float16).astype(np.float32))
    for x in rows:
        codes, sc = Q.quantize_rows_int8(x, "f32")
        t = torch.from_numpy(x)
        ts = t.abs().amax(dim=-1) / torch.tensor(127.0, dtype=torch.float32)
        tq = torch.clamp(torch.round(t / ts[:, None]), -127, 127).to(torch.int64)
        assert np.array_equal(sc, ts.numpy())
        assert np.array_equal(Q.decode(codes, "int8").astype(np.int64), tq.numpy())


def _token_pools(seed, NB, Hkv, bs, D):
    """int8 code pools and per-row power-of-two scales, and the float32 pools of the values
    they stand for (exact)."""
    from oracle import quant as Q
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 256, size=(NB, Hkv, bs, D)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(NB, Hkv, D, bs)).astype(np.uint8)
    ks = (2.0 ** rng.integers(-9, -4, size=(NB, Hkv, bs))).astype(np.float32)
    vs = (2.0 ** rng.integers(-9, -4, size=(NB, Hkv, bs))).astype(np.float32)
    kf = (Q.decode(kc, "int8") * ks[..., None]).astype(np.float32)
    vf = (Q.decode(vc, "int8") * vs[:, :, None, :]).astype(np.float32)
    return kc, vc, ks, vs, kf, vf


def check_int8_token_attention_lossless(seed=57):
    """Attention over int8 pools with a scale per (token, KV head) equals attention over the
    float32 pools holding exactly code * scale of each row: MHA and GQA, permuted tables,
    a mask, and every row of decode_one."""
    from oracle import quant as Q
    for S, H, Hkv, D, bs in ((3, 8, 2, 32, 16), (2, 4, 4, 64, 32)):
        NB = 12
        kc, vc, ks, vs, kf, vf = _token_pools(seed + H, NB, Hkv, bs, D)
        rng = np.random.default_rng(seed)
        tables = np.stack([rng.permutation(NB)[:4] for _ in range(S)]).astype(np.int32)
        ctx = [1, 3 * bs + 5, 4 * bs][:S]
        q = normal_host((S, H, D), seed + 1, "f32")
        quant = (Q.INT8_TOKEN, ks, vs)
        want = A.paged_decode(q, kf, vf, tables, ctx, 0.3, "f32")
        got = A.paged_decode(q, kc, vc, tables, ctx, 0.3, "f32", quant=quant)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
        lo, hi = [0] * S, [min(9, c) for c in ctx]
        want = A.paged_decode(q, kf, vf, tables, ctx, 0.3, "f32", masks=(lo, hi))
        got = A.paged_decode(q, kc, vc, tables, ctx, 0.3, "f32", quant=quant, masks=(lo, hi))
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
        full = A.paged_decode(q, kc, vc, tables, ctx, 0.3, "f32", quant=quant)
        for s in range(S):
            for h in range(H):
                row = A.decode_one(q[s], kc, vc, tables[s], ctx[s], h, H, 0.3, "f32", quant=quant)
                assert np.array_equal(row, full[s, h]), (s, h)


def check_int8_token_write_round_trip(seed=59):
    """The per-row quantising write: every written row reads back within half a code step of
    its input, with its scale at (block, KV head, offset) of the scale arrays and its largest
    element at +-127; slots < 0 and every other row and scale are left as they were."""
    from oracle import quant as Q
    NB, Hkv, bs, D = 6, 2, 16, 32
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 256, size=(NB, Hkv, bs, D)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(NB, Hkv, D, bs)).astype(np.uint8)
    ks = rng.uniform(0.01, 0.1, size=(NB, Hkv, bs)).astype(np.float32)
    vs = rng.uniform(0.01, 0.1, size=(NB, Hkv, bs)).astype(np.float32)
    T = 5
    key = normal_host((T, Hkv, D), seed + 1, "bf16")
    val = normal_host((T, Hkv, D), seed + 2, "bf16")
    slots = np.array([3, 17, -1, 95, 40], dtype=np.int32)
    kc2, vc2, ks2, vs2 = C.reshape_and_cache_int8_token(key, val, kc, vc, ks, vs, slots, "bf16")
    touched = np.zeros((NB, bs), bool)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        b, o = divmod(int(slot), bs)
        touched[b, o] = True
        for h in range(Hkv):
            for rows, codes, scale in ((key, kc2[b, h, o], ks2[b, h, o]), (val, vc2[b, h, :, o], vs2[b, h, o])):
                x = A.to_f64(rows[i, h], "bf16")
                got = Q.decode(codes, "int8") * float(scale)
                assert np.max(np.abs(got - x)) <= 0.50001 * float(scale)
                assert np.max(np.abs(Q.decode(codes, "int8"))) == 127.0
    for b in range(NB):
        for o in range(bs):
            if not touched[b, o]:
                assert np.array_equal(kc2[b, :, o], kc[b, :, o]) and np.array_equal(vc2[b, :, :, o], vc[b, :, :, o])
                assert np.array_equal(ks2[b, :, o], ks[b, :, o]) and np.array_equal(vs2[b, :, o], vs[b, :, o])


TOKEN_PINS = [check_int8_rows_closed_forms, check_int8_rows_vs_torch, check_int8_token_attention_lossless,
              check_int8_token_write_round_trip]



# ----------------------------------------------------------------------------
# prefix caching ("PagedAttention 实现细节" §3.2)

def check_p4_prefix_demo():
    """The page's demo, run through the allocator: blocks in use without and with the
    prefix cache, the saving, the one prompt evaluation, the hole, and the teardown."""
    g = golden("p4_prefix_demo.json")
    R, bs = g["num_requests"], g["block_size"]
    NB = 4 * R * (g["prefix_blocks"] + g["user_blocks"])
    system = list(range(1000, 1000 + g["system_tokens"]))

    plain = AL.BlockAllocator(NB, bs)
    for r in range(R):
        plain.seq_create(r, g["system_tokens"] + g["user_tokens"])
    without = NB - plain.num_free_blocks()
    assert without == g["blocks_without_cache"]

    al = AL.BlockAllocator(NB, bs)
    misses, pids = 0, set()
    for r in range(R):
        pid, hit = al.prefix_get_or_create(system)
        misses += 0 if hit else 1
        pids.add(pid)
        al.seq_create_with_prefix(r, pid, g["user_tokens"])
    with_cache = NB - al.num_free_blocks()
    assert with_cache == g["blocks_with_cache"]
    assert misses == g["prompt_evaluations_with_cache"] and len(pids) == 1
    saved = without - with_cache
    assert saved == g["blocks_saved"]
    assert f"{saved / without * 100:.1f}" == g["saving_percent"]
    assert f"{saved * g['kib_per_block'] / 1024:.1f}" == g["saved_mib"]
    (pid,) = pids
    blocks, length, users = al.prefix_info(pid)
    assert len(blocks) == g["prefix_blocks"] and length == g["system_tokens"] and users == R
    assert al.ref_count(blocks[0]) == 1 + R          # the entry's reference and one per request
    for r in range(R):
        t = al.block_table(r)
        assert t[0] == blocks[0] and len(t) == g["prefix_blocks"] + g["user_blocks"]
    # the request's own tokens start at the next block: positions 9..15 are a hole
    assert al.seq_len(0) == g["prefix_blocks"] * bs + g["user_tokens"]
    assert al.masks([0]) == ([g["system_tokens"]], [g["prefix_blocks"] * bs])
    slot, src, dst = al.seq_append_slot(0)          # the next token goes after the own tokens
    assert (src, dst) == (-1, -1)
    assert slot == al.block_table(0)[(bs + g["user_tokens"]) // bs] * bs + (bs + g["user_tokens"]) % bs
    # teardown: every request leaves; the entry goes with its last user
    for r in range(R):
        al.seq_free(r)
        al.prefix_release(pid)
    assert al.num_free_blocks() == NB and all(c == 0 for c in al.refs)
    _, hit = al.prefix_get_or_create(system)
    assert not hit


# ----------------------------------------------------------------------------
# masked positions (prefix hole, sliding window)

def check_masked_against_sdpa(seed=61, S=4, H=8, Hkv=2, D=32, bs=16):
    """Masked decode equals torch's SDPA on the contiguous cache with the masked rows
    removed (independent of the oracle's gather), for a prefix hole, a sliding window, an
    empty mask and a mask covering everything (zero row)."""
    import torch
    import torch.nn.functional as F

    ctx = (46, 90, 33, 20)
    q, kc, vc, tables, ctx, Ks, Vs = scatter_case(seed, S, H, Hkv, D, bs, ctx, "f32")
    lo = [9, 0, 5, 0]            # hole [9, 16); window of the last 24; [5, 5) empty; all masked
    hi = [16, 90 - 24, 5, 20]
    scale = 1.0 / math.sqrt(D)
    out = A.paged_decode(q, kc, vc, tables, ctx, scale, "f32", masks=(lo, hi))
    for s in range(S):
        keep = [t for t in range(ctx[s]) if not lo[s] <= t < hi[s]]
        if not keep:
            assert np.array_equal(out[s], np.zeros((H, D)))
            continue
        qt = torch.from_numpy(A.to_f64(q[s], "f32")).view(1, H, 1, D)
        kt = torch.from_numpy(Ks[s][:, keep]).view(1, Hkv, len(keep), D)
        vt = torch.from_numpy(Vs[s][:, keep]).view(1, Hkv, len(keep), D)
        ref = F.scaled_dot_product_attention(qt, kt, vt, scale=float(np.float32(scale)),
                                             enable_gqa=True).view(H, D).numpy()
        assert np.max(np.abs(out[s] - ref)) <= 1e-12, f"seq {s}"


def check_masked_split_merge(seed=67, n=700, D=16):
    """Masked partials merge to the masked direct result for any partition size; a partition
    wholly inside the mask is (-inf, 0, 0); everything masked merges to zeros."""
    rng = np.random.default_rng(seed)
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    scale = 0.3
    for lo, hi in ((100, 480), (0, 650), (9, 16), (0, 0)):
        keep = [t for t in range(n) if not lo <= t < hi]
        direct = A.attend(q, K[keep], V[keep], scale)
        for ps in (16, 100, 512):
            m, l, o = A.partition_partials(q, K[keep], V[keep], scale, ps, keep, n)
            assert np.max(np.abs(A.lse_merge(m, l, o) - direct)) <= 1e-12, (lo, hi, ps)
            for p in range(len(m)):
                if all(lo <= t < hi for t in range(p * ps, min((p + 1) * ps, n))):
                    assert m[p] == -np.inf and l[p] == 0 and not o[p].any()
    m, l, o = A.partition_partials(q, K[:0], V[:0], scale, 64, [], n)
    assert np.array_equal(A.lse_merge(m, l, o), np.zeros(D))


MASK_PINS = [check_masked_against_sdpa, check_masked_split_merge]


# ----------------------------------------------------------------------------
# several query tokens per sequence

def check_multi_against_sdpa(seed=71, H=8, Hkv=2, D=32, bs=16):
    """Each sequence's span of query tokens against torch's float64 SDPA with an explicit
    boolean mask (key t allowed for query i iff t <= n - L + i), on the contiguous cache."""
    import torch
    import torch.nn.functional as F

    ctx = (40, 7, 100, 16)
    spans = (4, 1, 7, 16)            # the last span covers the whole context
    q, kc, vc, tables, ctx, Ks, Vs = scatter_case(seed, len(ctx), H, Hkv, D, bs, ctx, "f32")
    qstart = np.concatenate([[0], np.cumsum(spans)]).astype(np.int32)
    qm = normal_host((int(qstart[-1]), H, D), seed + 9, "f32")
    scale = 0.2
    out = A.paged_decode_multi(qm, kc, vc, tables, ctx, qstart, scale, "f32")
    for s, (n, L) in enumerate(zip(ctx, spans)):
        rows = slice(int(qstart[s]), int(qstart[s + 1]))
        qt = torch.from_numpy(qm[rows].astype(np.float64)).permute(1, 0, 2).unsqueeze(0)   # [1, H, L, D]
        kt = torch.from_numpy(Ks[s]).unsqueeze(0)
        vt = torch.from_numpy(Vs[s]).unsqueeze(0)
        allowed = torch.tensor([[t <= n - L + i for t in range(n)] for i in range(L)])
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=float(np.float32(scale)),
                                             enable_gqa=True)
        ref = ref.squeeze(0).permute(1, 0, 2).numpy()
        assert np.max(np.abs(out[rows] - ref)) <= 1e-12, f"seq {s}"


def check_multi_reduces_to_decode(seed=73):
    """One query token per sequence is plain decode; the last token of any span sees the
    whole context, so it equals plain decode of that token."""
    H, Hkv, D, bs = 4, 4, 16, 16
    ctx = (1, 30, 64)
    q, kc, vc, tables, ctx, _, _ = scatter_case(seed, 3, H, Hkv, D, bs, ctx, "f32")
    ones = np.arange(4, dtype=np.int32)
    assert np.array_equal(A.paged_decode_multi(q, kc, vc, tables, ctx, ones, 0.25, "f32"),
                          A.paged_decode(q, kc, vc, tables, ctx, 0.25, "f32"))
    spans = (1, 5, 9)
    qstart = np.concatenate([[0], np.cumsum(spans)]).astype(np.int32)
    qm = normal_host((int(qstart[-1]), H, D), seed + 1, "f32")
    out = A.paged_decode_multi(qm, kc, vc, tables, ctx, qstart, 0.25, "f32")
    last = qm[qstart[1:] - 1]
    assert np.array_equal(out[qstart[1:] - 1], A.paged_decode(last, kc, vc, tables, ctx, 0.25, "f32"))


MULTI_PINS = [check_multi_against_sdpa, check_multi_reduces_to_decode]


# ----------------------------------------------------------------------------
# swap to the host pool, sliding-window release

def _logical(al, pools, s):
    """Token data of sequence s read through its table from the pool it lives in
    (pools = {"dev": array [NB, bs], "host": array [NH, bs]})."""
    pool = pools["host"] if s in al.swapped else pools["dev"]
    bs = al.block_size
    return [pool[al.tables[s][t // bs], t % bs] for t in range(al.lens[s])]


def check_swap_round_trip(seed=81):
    """Swapping a group out and back in keeps every sequence's token data (the copy pairs,
    applied as whole-block copies between the pools, move exactly what the tables need),
    keeps sharing inside the group, returns the group's device blocks while it is out and
    takes the host blocks back afterwards."""
    rng = np.random.default_rng(seed)
    NB, NH, bs = 40, 24, 4
    al = AL.BlockAllocator(NB, bs, rng.permutation(NB))
    al.set_host_pool(NH)
    al.seq_create(1, 10)
    al.seq_fork(1, 2, 9)                 # shares 3 blocks with 1
    al.seq_append_slot(2)                # copy-on-write of the shared last block
    al.seq_create(3, 7)
    al.seq_fork(3, 4)                    # 4 shares with 3, which stays on the device
    pools = {"dev": rng.integers(0, 10**6, size=(NB, bs)), "host": np.full((NH, bs), -1)}
    before = {s: _logical(al, pools, s) for s in (1, 2, 3, 4)}
    free0 = al.num_free_blocks()
    distinct = len({b for s in (1, 2, 4) for b in al.tables[s]})
    private = len({b for s in (1, 2, 4) for b in al.tables[s]} - set(al.tables[3]))
    pairs = al.seq_swap_out([1, 2, 4])
    assert len(pairs) == distinct and len({d for d, _ in pairs}) == distinct
    for d, h in pairs:
        pools["host"][h] = pools["dev"][d]
    assert al.num_free_blocks() == free0 + private
    assert len(al.host_free_list()) == NH - distinct
    assert all(al.ref_count(b) == 1 for b in al.tables[3])       # 4's references left with it
    assert al.tables[1][:2] == al.tables[2][:2]                     # still shared, now on the host
    assert al.host_refs[al.tables[1][0]] == 2
    for s in (1, 2, 3, 4):
        assert _logical(al, pools, s) == before[s]
    # the freed device blocks may be reused meanwhile
    al.seq_create(5, 4 * al.num_free_blocks() - 8)
    pools["dev"][al.tables[5]] = -7
    al.seq_free(5)
    pairs = al.seq_swap_in([2, 1, 4])
    for h, d in pairs:
        pools["dev"][d] = pools["host"][h]
    assert len(al.host_free_list()) == NH
    for s in (1, 2, 3, 4):
        assert _logical(al, pools, s) == before[s]
    assert al.tables[1][:2] == al.tables[2][:2] and al.ref_count(al.tables[1][0]) == 2
    assert al.ref_count(al.tables[4][0]) == 1 and al.tables[4][0] != al.tables[3][0]


def check_swap_blocks(seed=83):
    """The pool-to-pool copy: swapping a group out to a host pool and back into other device
    blocks returns each sequence's logical contents unchanged; blocks no pair names keep their
    bytes; between two halves of one pool it is the in-pool block copy."""
    rng = np.random.default_rng(seed)
    NB, NH, Hkv, bs, D = 12, 6, 2, 16, 8
    kc = normal_host((NB, Hkv, bs, D), seed, "f16")
    vc = normal_host((NB, Hkv, D, bs), seed + 1, "f16")
    hk = np.zeros((NH, Hkv, bs, D), np.float16)
    hv = np.zeros((NH, Hkv, D, bs), np.float16)
    out_pairs = [(3, 0), (7, 4), (11, 2)]
    hk2, hv2 = C.swap_blocks(hk, hv, kc, vc, out_pairs)
    for d, h in out_pairs:
        assert np.array_equal(hk2[h], kc[d]) and np.array_equal(hv2[h], vc[d])
    for h in (1, 3, 5):
        assert not hk2[h].any() and not hv2[h].any()
    in_pairs = [(0, 9), (4, 1), (2, 5)]
    kc2, vc2 = C.swap_blocks(np.zeros_like(kc), np.zeros_like(vc), hk2, hv2, in_pairs)
    moved = {3: 9, 7: 1, 11: 5}
    for d0, d1 in moved.items():
        assert np.array_equal(kc2[d1], kc[d0]) and np.array_equal(vc2[d1], vc[d0])
    pairs = [(int(a), int(b)) for a, b in zip(rng.permutation(6), rng.permutation(6) + 6)]
    ek, ev = C.copy_blocks(kc, vc, pairs)
    gk, gv = C.swap_blocks(kc, vc, kc.copy(), vc.copy(), pairs)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


def check_window_release():
    """A window of W keeps the blocks holding positions >= len - W: closed-form tables,
    free counts and masks as the sequence grows."""
    bs, W = 16, 40
    al = AL.BlockAllocator(64, bs)
    al.seq_create(1, 100)                # blocks 0..6, positions 0..99
    t0 = list(al.tables[1])
    al.seq_set_window(1, W)              # start 60: blocks 0..2 (positions 0..47) released
    assert al.tables[1] == [-1, -1, -1] + t0[3:]
    assert al.num_free_blocks() == 64 - 7 + 3
    assert al.masks([1]) == ([0], [60])
    for _ in range(20):                  # len 120, start 80: block 3 (48..63) and 4 (64..79) released
        al.seq_append_slot(1)
    assert al.tables[1][:5] == [-1] * 5 and all(b >= 0 for b in al.tables[1][5:])
    assert len(al.tables[1]) == 8 and al.masks([1]) == ([0], [80])
    assert al.num_free_blocks() == 64 - 3


def _check_window_fork():
    bs, W = 16, 40
    al = AL.BlockAllocator(64, bs)
    al.seq_create(1, 120)
    al.seq_set_window(1, W)              # start 80: blocks 0..4 dropped
    try:
        al.seq_fork(1, 2, 110)           # start 70 needs block 4
    except AL.AllocatorError as e:
        assert e.code == AL.INVALID_ARG
    else:
        raise AssertionError("fork into dropped blocks must fail")
    al.seq_fork(1, 3, 120)
    assert al.tables[3] == al.tables[1] and al.masks([3]) == ([0], [80])
    assert all(al.ref_count(b) == 2 for b in al.tables[1] if b >= 0)
    al.seq_free(1)
    al.seq_free(3)
    assert al.num_free_blocks() == 64


def check_window():
    check_window_release()
    _check_window_fork()


SWAP_WINDOW_PINS = [check_swap_round_trip, check_window]
