"""GPU parity of decode with several causal query tokens per sequence (pa_decode_multi, the
verification pass of speculative decoding) against the float64 oracle: every model dtype
and both 8-bit formats, head groups from 1 to 8 (tiles of heads x query tokens), spans
from 0 to the whole context, several workgroups per span, single pass and split; one
token per sequence is bit-identical to pa_decode; a span longer than its context gives
NaN rows.  Unused rows of the pools are poisoned.  Tolerances as in tests/gpu_helpers.py."""
import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_333_amd as pa
import synth
from oracle import attention as A
from tests.gpu_helpers import DeviceWorkload, assert_close, out_to_f64, scale_for

pytestmark = pytest.mark.gpu

KINDS = [("f32", None), ("f16", None), ("bf16", None), ("f16", "fp8_e4m3"), ("bf16", "int8")]
# (element type, 8-bit format, head_dim, block size); 8-bit pools take no 8-token blocks (the host
# rejects them, tested on the CPU)
POOL_CASES = [(dt, fmt, D, bs) for D, bs in [(64, 16), (128, 32), (128, 16), (128, 8), (128, 64)]
              for dt, fmt in KINDS if not (fmt and bs == 8)]
POISON_CODE = {"fp8_e4m3": 0x7F, "int8": 0x80}


def make_case(seed, dt, fmt, H, Hkv, D, bs, ctx, spans, poison=True):
    rng = np.random.default_rng(seed)
    S = len(ctx)
    need = [-(-n // bs) for n in ctx]
    NB = sum(need) + 4
    MB = max(need + [1]) + 1
    perm = rng.permutation(NB)
    tables = -np.ones((S, MB), dtype=np.int32)
    pos = 0
    for s in range(S):
        tables[s, :need[s]] = perm[pos:pos + need[s]]
        pos += need[s]
    if fmt:
        kc = synth.normal_codes_host((NB, Hkv, bs, D), seed + 1, fmt)
        vc = synth.normal_codes_host((NB, Hkv, D, bs), seed + 2, fmt)
    else:
        kc = synth.normal_host((NB, Hkv, bs, D), seed + 1, dt)
        vc = synth.normal_host((NB, Hkv, D, bs), seed + 2, dt)
    qstart = np.concatenate([[0], np.cumsum(spans)]).astype(np.int32)
    T = int(qstart[-1])
    q = synth.normal_host((T, H, D), seed + 3, dt)
    if poison:
        used = np.zeros((NB, bs), dtype=bool)
        for s in range(S):
            for t in range(ctx[s]):
                used[tables[s, t // bs], t % bs] = True
        bad = POISON_CODE[fmt] if fmt else \
            {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dt]
        for b in range(NB):
            for o in range(bs):
                if not used[b, o]:
                    kc[b, :, o, :] = bad
                    vc[b, :, :, o] = bad
    ks, vs = (float(np.float32(1.1 / synth.CODE_SIGMA[fmt])), float(np.float32(0.9 / synth.CODE_SIGMA[fmt]))) \
        if fmt else (1.0, 1.0)
    return dict(q=q, kc=kc, vc=vc, tables=tables, ctx=list(ctx), qstart=qstart, spans=list(spans), NB=NB, MB=MB,
                dt=dt, fmt=fmt, S=S, T=T, H=H, Hkv=Hkv, D=D, bs=bs, ks=ks, vs=vs)


def dev(c):
    d = "cuda"
    if c["fmt"]:
        kc, vc = torch.from_numpy(c["kc"]).to(d), torch.from_numpy(c["vc"]).to(d)
    else:
        kc, vc = synth.to_torch(c["kc"], c["dt"]).to(d), synth.to_torch(c["vc"], c["dt"]).to(d)
    return dict(q=synth.to_torch(c["q"], c["dt"]).to(d), kc=kc, vc=vc, tab=torch.from_numpy(c["tables"]).to(d),
                ctx=torch.tensor(c["ctx"], dtype=torch.int32, device=d),
                qst=torch.from_numpy(c["qstart"]).to(d))


def run(c, dv, split=None, max_q=None, order=None):
    max_q = max(c["spans"] + [1]) if max_q is None else max_q
    max_ctx = c["MB"] * c["bs"]
    ws = None
    if split:
        ws = torch.empty(pa.pa_decode_multi_workspace_bytes(c["T"], c["H"], c["D"], max_ctx, split),
                         dtype=torch.uint8, device="cuda")
    so = None if order is None else torch.tensor(order, dtype=torch.int32, device="cuda")
    out = torch.full_like(dv["q"], 7.0)
    path = pa.pa_decode_multi(out, dv["q"], dv["kc"], dv["vc"], dv["tab"], dv["ctx"], dv["qst"], max_q, max_ctx,
                              scale_for(c["D"]), c["ks"], c["vs"], kv_format=c["fmt"], partition_size=split or 512,
                              workspace=ws, split=split is not None, seq_order=so)
    torch.cuda.synchronize()
    assert path == ("single" if split is None else "split")
    return out_to_f64(out, c["dt"])


def oracle(c):
    quant = (c["fmt"], c["ks"], c["vs"]) if c["fmt"] else None
    return A.paged_decode_multi(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], c["qstart"], scale_for(c["D"]),
                                c["dt"], quant=quant)


CTX = (1, 17, 40, 100, 64, 33, 16, 90)
SPANS = (1, 1, 4, 7, 16, 3, 16, 0)   # one token, a few, a full tile, the whole context, none


@pytest.mark.parametrize("dt,fmt,D,bs", POOL_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 2), (16, 2), (6, 2), (32, 2)])
def test_multi_families(dt, fmt, D, bs, H, Hkv):
    c = make_case(zlib.crc32(repr((dt, fmt, D, bs, H, Hkv)).encode()) % 10000, dt, fmt, H, Hkv, D, bs, CTX, SPANS)
    dv = dev(c)
    ref = oracle(c)
    single = run(c, dv)
    assert_close(single, ref, dt, "single pass")
    for ps in (2 * bs, 64):
        assert_close(run(c, dv, split=ps), ref, dt, f"split {ps}")
    order = pa.pa_order_longest_first(list(CTX))
    assert np.array_equal(run(c, dv, order=order), single)
    # a larger max_query_len bound only adds empty workgroups
    assert np.array_equal(run(c, dv, max_q=40), single)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_multi_long_spans_take_several_workgroups(dt):
    """Spans of 37 and 64 tokens (several tiles per sequence and head group) and long contexts."""
    c = make_case(5, dt, None, 8, 2, 128, 16, (2000, 64, 777), (37, 64, 5))
    dv = dev(c)
    ref = oracle(c)
    assert_close(run(c, dv), ref, dt, "single pass")
    assert_close(run(c, dv, split=512), ref, dt, "split 512")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_one_token_per_sequence_is_bit_identical_to_decode(dt):
    ctx = (1, 17, 40, 100, 64, 33)
    c = make_case(9, dt, None, 8, 2, 128, 16, ctx, (1,) * 6)
    dv = dev(c)
    out = torch.empty_like(dv["q"])
    pa.pa_decode(out, dv["q"], dv["kc"], dv["vc"], dv["tab"], dv["ctx"], c["MB"] * c["bs"], scale_for(128))
    torch.cuda.synchronize()
    assert np.array_equal(run(c, dv), out_to_f64(out, dt))


def test_span_longer_than_context_gives_nan_rows():
    c = make_case(13, "f16", None, 4, 4, 64, 16, (10, 30), (12, 3), poison=False)
    dv = dev(c)
    got = run(c, dv)
    assert np.all(np.isnan(got[:12]))
    ok = A.paged_decode_multi(c["q"][12:], c["kc"], c["vc"], c["tables"][1:], [30], np.array([0, 3]),
                              scale_for(64), "f16")
    assert_close(got[12:], ok, "f16", "the valid sequence")


def test_speculative_verification_full_size_every_row():
    """LLaMA-7B-like layer (64 sequences, 32 heads, fp16): the last 4 tokens of every sequence
    verified in one launch, the one the bench times; every row against the oracle."""
    dw = DeviceWorkload(2)
    w = dw.w
    L = 4
    T = w.num_seqs * L
    q = synth.normal_device((T, w.num_heads, w.head_dim), 4242, w.dtype)
    qst = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.empty(pa.pa_decode_multi_workspace_bytes(T, w.num_heads, w.head_dim, dw.max_context_len, 512),
                     dtype=torch.uint8, device="cuda")
    path = pa.pa_decode_multi(out, q, dw.key_cache, dw.value_cache, dw.tables, dw.context_lens, qst, L,
                              dw.max_context_len, w.scale, partition_size=512, workspace=ws)
    torch.cuda.synchronize()
    assert path == "single"
    got = out_to_f64(out, w.dtype)
    qn = synth.to_numpy(q, w.dtype)
    _, kc, vc, tabs, lens = dw.oracle_inputs()
    ref = A.paged_decode_multi(qn, kc, vc, tabs, lens, qst.cpu().numpy(), w.scale, w.dtype)
    assert_close(got, ref, w.dtype, "verification of 4 tokens, every row")
