"""GPU parity of pa_decode_append: the slot-mapping write fused into decode.

It must equal pa_reshape_and_cache followed by the same decode path, bit for bit
(pools and outputs), and match the float64 oracle on the pools after the write
(oracle/cache_ops.reshape_and_cache) within the decode tolerance."""
import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_333_amd as pa
import synth
from oracle import attention as A
from oracle import cache_ops as C
from tests.gpu_helpers import DeviceWorkload, assert_close, out_to_f64, scale_for
from tests.test_gpu_decode import make_case, to_dev

pytestmark = pytest.mark.gpu


def bits(a):
    """Storage bit patterns, so NaN-poisoned pools compare exactly."""
    a = np.ascontiguousarray(a)
    return a.view({4: np.uint32, 2: np.uint16}[a.dtype.itemsize])


def _new_tokens(c, seed):
    """New K/V rows for each sequence and the slot of its last token (position ctx-1).
    Sequences with an empty context get slot -1 except the first, which gets a free slot
    (written although nothing reads it)."""
    S, Hkv, D, bs = c["S"], c["Hkv"], c["D"], c["bs"]
    key = synth.normal_host((S, Hkv, D), seed + 7, c["dtype"])
    val = synth.normal_host((S, Hkv, D), seed + 8, c["dtype"])
    slots = np.full(S, -1, dtype=np.int32)
    used = set(int(b) for b in c["tables"].ravel() if b >= 0)
    free = [b for b in range(c["NB"]) if b not in used]
    first_empty = True
    for s, n in enumerate(c["ctx"]):
        if n > 0:
            p = n - 1
            slots[s] = c["tables"][s, p // bs] * bs + p % bs
        elif first_empty and free:
            slots[s] = free[0] * bs + 3 % bs
            first_empty = False
    return key, val, slots


def _run_both(c, key, val, slots, split_ps=None):
    """(fused out, fused pools) and (separate out, separate pools) on fresh device copies."""
    res = []
    for fused in (True, False):
        dv = to_dev(c)
        dk, dvv = synth.to_torch(key, c["dtype"]).cuda(), synth.to_torch(val, c["dtype"]).cuda()
        ds = torch.from_numpy(slots).cuda()
        out = torch.full_like(dv["q"], 7.0)
        max_ctx = c["MB"] * c["bs"]
        ws = None
        if split_ps:
            ws = torch.empty(pa.pa_decode_split_workspace_bytes(c["S"], c["H"], c["D"], max_ctx, split_ps),
                             dtype=torch.uint8, device="cuda")
        scale = scale_for(c["D"])
        if fused:
            path = pa.pa_decode_append(out, dv["q"], dk, dvv, ds, dv["kc"], dv["vc"], dv["tables"], dv["ctx"],
                                       max_ctx, scale, split_ps or 512, ws)
        else:
            pa.pa_reshape_and_cache(dk, dvv, dv["kc"], dv["vc"], ds)
            path = pa.pa_decode_auto(out, dv["q"], dv["kc"], dv["vc"], dv["tables"], dv["ctx"], max_ctx, scale,
                                     split_ps or 512, ws)
        torch.cuda.synchronize()
        res.append((out.clone(), synth.to_numpy(dv["kc"], c["dtype"]), synth.to_numpy(dv["vc"], c["dtype"]), path))
    return res


FAMILIES = [(dt, D, bs, H, Hkv) for dt in ("f32", "f16", "bf16") for D in (64, 128) for bs in (16, 32)
            for (H, Hkv) in ((4, 4), (16, 4), (16, 1), (32, 1))]
FAMILIES += [(dt, 128, bs, H, Hkv) for dt in ("f32", "f16", "bf16") for bs in (8, 64)
             for (H, Hkv) in ((4, 4), (16, 1))]


@pytest.mark.parametrize("dt,D,bs,H,Hkv", FAMILIES, ids=lambda v: str(v))
def test_append_equals_write_then_decode(dt, D, bs, H, Hkv):
    # ragged contexts that already count the new token; unused rows poisoned with NaN
    ctx = (1, bs, bs + 1, 3 * bs + 5, 0, 7 * bs)
    seed = zlib.crc32(repr((dt, D, bs, H, Hkv)).encode()) % 10000
    c = make_case(seed, dt, len(ctx), H, Hkv, D, bs, ctx, poison=True)
    key, val, slots = _new_tokens(c, seed)
    ek, ev = C.reshape_and_cache(key, val, c["kc"], c["vc"], slots)
    ref = A.paged_decode(c["q"], ek, ev, c["tables"], c["ctx"], scale_for(D), dt)
    for split_ps in (None, 2 * bs):
        (fo, fk, fv, fpath), (so, sk, sv, spath) = _run_both(c, key, val, slots, split_ps)
        assert fpath == spath == ("single" if split_ps is None else "split")
        assert np.array_equal(bits(fk), bits(ek)) and np.array_equal(bits(fv), bits(ev)), "pools after the write"
        assert np.array_equal(bits(sk), bits(ek)) and np.array_equal(bits(sv), bits(ev))
        assert torch.equal(fo, so), f"fused differs from write-then-decode ({fpath})"
        assert_close(out_to_f64(fo, dt), ref, dt, f"fused {fpath}")


def test_append_negative_slot_writes_nothing():
    c = make_case(3, "f16", 2, 8, 2, 128, 16, (20, 33))
    key, val, slots = _new_tokens(c, 3)
    slots[:] = -1
    (fo, fk, fv, _), (so, _, _, _) = _run_both(c, key, val, slots)
    assert np.array_equal(bits(fk), bits(c["kc"])) and np.array_equal(bits(fv), bits(c["vc"]))
    assert torch.equal(fo, so)


@pytest.mark.parametrize("key", [2, 3])
def test_append_full_size_step(key):
    """A full LLaMA-7B-like / GQA step: the allocator reserves one slot per sequence and the
    fused call writes and decodes; it equals the separate calls bit for bit."""
    dw = DeviceWorkload(key)
    w = dw.w
    slots, pairs = dw.alloc.seq_append_slots(dw.seq_ids)
    assert not pairs
    dw.refresh_tables()
    nk = synth.normal_device((w.num_seqs, w.num_kv_heads, w.head_dim), dw.seeds["new_key"], w.dtype)
    nv = synth.normal_device((w.num_seqs, w.num_kv_heads, w.head_dim), dw.seeds["new_value"], w.dtype)
    ds = torch.tensor(slots, dtype=torch.int32, device="cuda")
    order = torch.tensor(pa.pa_order_longest_first(list(dw.ora.lens[s] + 1 for s in dw.seq_ids)),
                         dtype=torch.int32, device="cuda")
    kc0, vc0 = dw.key_cache.clone(), dw.value_cache.clone()
    pa.pa_decode_append(dw.out, dw.query, nk, nv, ds, dw.key_cache, dw.value_cache, dw.tables, dw.context_lens,
                        dw.max_context_len, w.scale, seq_order=order)
    fused = dw.out.clone()
    kc1, vc1 = dw.key_cache.clone(), dw.value_cache.clone()
    dw.key_cache.copy_(kc0)
    dw.value_cache.copy_(vc0)
    pa.pa_reshape_and_cache(nk, nv, dw.key_cache, dw.value_cache, ds)
    pa.pa_decode(dw.out, dw.query, dw.key_cache, dw.value_cache, dw.tables, dw.context_lens, dw.max_context_len,
                 w.scale, seq_order=order)
    torch.cuda.synchronize()
    assert torch.equal(kc1, dw.key_cache) and torch.equal(vc1, dw.value_cache)
    assert torch.equal(fused, dw.out)
