"""Each workload's decode step exactly as bench.py runs it, against the oracle on every output row.

Bench.step is called itself, once, from the workload's initial state: the C++ allocator's
append (copy-on-write pairs for the parallel-sampling workload), the upload of the step's
index data, the block copies, the new-token write (quantising for the 8-bit pools) and the
decode call the bench times (single pass, split + merge, shared prefix, four verified query
tokens).  The oracle side builds its own allocator from the workload's definition, appends
the same tokens, copies and writes into host copies of the pre-step blocks, and decodes from
those; no oracle input comes from a kernel of the library.  The step's index data must equal
the oracle allocator's, the blocks the step touched or reads must equal the oracle's copy and
write bit for bit, and every output row must match the oracle's decode ("PagedAttention
实现细节" §3.3, the copy-on-write timeline; §3.4, the write after each step)."""
import numpy as np
import pytest
import torch

import bench
import synth
from oracle import allocator as AL
from oracle import attention as A
from oracle import cache_ops as OC
from tests.gpu_helpers import (assert_close, fetch_blocks, fetch_token_blocks, out_to_f64, renumber, renumber_slots,
                               used_blocks)

pytestmark = pytest.mark.gpu

BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def oracle_allocator(w):
    """The workload's initial allocator state, built by the oracle allocator."""
    al = AL.BlockAllocator(w.num_blocks, w.block_size, w.free_order)
    if w.key == 5:
        for g in range(w.groups):
            parent = 10_000 + g
            al.seq_create(parent, w.parent_len)
            for b in range(w.branches):
                s = g * w.branches + b
                al.seq_fork(parent, s, w.context_lens[s])
            al.seq_free(parent)
    else:
        for s, n in enumerate(w.context_lens):
            al.seq_create(s, n)
    return al


def same_bits(a, b, dtype, quant):
    if quant:
        return np.array_equal(a, b)
    return np.array_equal(a.view(BITS[dtype]), b.view(BITS[dtype]))


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_bench_step_every_row(key):
    print(f"bench step, workload {key}", flush=True)
    args = bench.parse(["--workload", str(key), "--steps", "1", "--warmup", "0", "--no-cpu-baseline"])
    b = bench.Bench(args)
    w = b.w
    S, L, bs = w.num_seqs, w.query_len, w.block_size
    quant = bool(w.kv_format)
    rows = w.kv_format == "int8_token"

    ora = oracle_allocator(w)
    slots, pairs = ora.seq_append_slots(list(range(S)) * L)
    tabs, lens = ora.build_block_tables(list(range(S)), b.max_blocks)
    if key == 5:
        assert len(pairs) > 0, "the parallel-sampling step copies shared last blocks"
    used = used_blocks(tabs, lens, bs, [x for p in pairs for x in p])

    def fetch_pools():
        if rows:
            kc, ks, vc, vs = fetch_token_blocks(b.kc, b.vc, used, bs, w.head_dim)
            return (kc, ks), (vc, vs)
        return fetch_blocks(b.kc, used, w.dtype, quant), fetch_blocks(b.vc, used, w.dtype, quant)

    kc0, vc0 = fetch_pools()

    b.step(0, None)
    torch.cuda.synchronize()

    buf = b.bufs[0]
    assert buf["slots_h"].tolist() == slots
    assert buf["pairs_h"][:len(pairs)].tolist() == [list(p) for p in pairs]
    assert buf["tab_h"].tolist() == tabs and buf["len_h"].tolist() == lens
    assert torch.equal(buf["idx_d"].cpu(), buf["idx_h"]), "the uploaded index data differs from the host's"

    nk = synth.to_numpy(b.newk[0], w.dtype)
    nv = synth.to_numpy(b.newv[0], w.dtype)
    pr = renumber(used, np.array(pairs, dtype=np.int64).reshape(-1)).reshape(-1, 2)
    rs = renumber_slots(used, slots, bs)
    kc1, vc1 = fetch_pools()
    if rows:
        (kc, ks), (vc, vs) = kc0, vc0
        kc, vc = OC.copy_blocks(kc, vc, pr)
        ks, vs = OC.copy_blocks(ks, vs, pr)
        kc, vc, ks, vs = OC.reshape_and_cache_int8_token(nk, nv, kc, vc, ks, vs, rs, w.dtype)
        assert np.array_equal(kc1[0], kc) and np.array_equal(vc1[0], vc), "codes after the step"
        assert np.array_equal(kc1[1].view(np.uint32), ks.view(np.uint32)), "key scales after the step"
        assert np.array_equal(vc1[1].view(np.uint32), vs.view(np.uint32)), "value scales after the step"
        qarg = (w.kv_format, ks, vs)
    else:
        kc, vc = OC.copy_blocks(kc0, vc0, pr)
        if quant:
            kc, vc = OC.reshape_and_cache_quant(nk, nv, kc, vc, rs, w.dtype, w.kv_format, w.k_scale, w.v_scale)
        else:
            kc, vc = OC.reshape_and_cache(nk, nv, kc, vc, rs)
        assert same_bits(kc1, kc, w.dtype, quant), "key pool after the step"
        assert same_bits(vc1, vc, w.dtype, quant), "value pool after the step"
        qarg = (w.kv_format, w.k_scale, w.v_scale) if quant else None

    q = synth.to_numpy(b.q, w.dtype)
    t2 = renumber(used, tabs)
    if L > 1:
        ref = A.paged_decode_multi(q, kc, vc, t2, lens, b.qstart.cpu().numpy(), w.scale, w.dtype)
    else:
        ref = A.paged_decode(q, kc, vc, t2, lens, w.scale, w.dtype, quant=qarg)
    path = "+".join(sorted(b.path_ran))
    assert_close(out_to_f64(b.out, w.dtype), ref, w.dtype, f"workload {key} bench step ({path}), every row")
    if key == 5:
        assert path == "shared"
    if key == 4:
        assert path == "split"
