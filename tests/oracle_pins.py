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
