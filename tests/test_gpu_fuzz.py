"""Seeded random cases across the decode calls' combinations, each against the oracle.

Every case draws its own dtype and pool format (fp32/fp16/bf16 pools, or FP8 E4M3 / int8
codes with per-pool scales under fp16/bf16 queries), head_dim, block size (8 and 64 only
with head_dim 128; 8-bit pools never with 8), KV heads and group size, batch, ragged
context lengths (empty, one token, block edges, several blocks), a shuffled block pool, and
one of the call paths: single pass, split at a random multiple of the block size, masked
(a random hole or window per sequence, single or split), or several causal query tokens
per sequence (single or split).  The tolerance is the parity tolerance of every other
decode test (tests/gpu_helpers.py).  The draws come from numpy PCG64 seeded by the case
number, so a failing case is reproduced by its id.

The first 64 cases run a second time with the softmax scale 40 times larger: logits of
tens to hundreds, so most weights underflow and the running maximum jumps between steps,
partitions and masked spans.  Their outputs approach single value rows, so fp16 and fp32
outputs there add half an ulp of the output type at |ref| (gpu_helpers.output_rounding_term,
included for bf16 everywhere), and fp32 outputs the error that rounding such logits to fp32
allows (gpu_helpers.fp32_logit_term, from the largest logit of the case)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_333_amd as pa
import synth
from oracle import attention as A
from tests.gpu_helpers import (assert_close, fp32_logit_term, max_abs_logit2, out_to_f64, output_rounding_term,
                               scale_for)

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = float(np.float32(0.0165)), float(np.float32(0.0145))
CASES = 256
WIDE_CASES, WIDE_GAIN = 64, 40.0


def draw(case):
    rng = np.random.default_rng(7000 + case)
    fmt = [None, None, None, "fp8_e4m3", "int8"][int(rng.integers(5))]
    dt = ["f16", "bf16"][int(rng.integers(2))] if fmt else ["f32", "f16", "bf16"][int(rng.integers(3))]
    D = int(rng.choice([64, 128]))
    sizes = [16, 32] + ([64] if D == 128 else []) + ([8] if D == 128 and not fmt else [])
    bs = int(rng.choice(sizes))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    S = int(rng.integers(1, 7))
    ctx = []
    for _ in range(S):
        kind = int(rng.integers(6))
        n = [0, 1, bs - 1, bs, bs + 1, int(rng.integers(2, 12 * bs))][kind]
        ctx.append(n)
    path = ["single", "split", "masked", "masked-split", "multi", "multi-split"][int(rng.integers(6))]
    ps = bs * int(rng.integers(1, 5))
    return rng, dict(fmt=fmt, dt=dt, D=D, bs=bs, Hkv=Hkv, H=Hkv * G, S=S, ctx=ctx, path=path, ps=ps)


def build(rng, c, seed):
    S, bs = c["S"], c["bs"]
    need = [-(-n // bs) for n in c["ctx"]]
    NB = sum(need) + 3
    MB = max(need + [1]) + 1
    perm = rng.permutation(NB)
    tables = -np.ones((S, MB), dtype=np.int32)
    pos = 0
    for s in range(S):
        tables[s, :need[s]] = perm[pos:pos + need[s]]
        pos += need[s]
    kshape, vshape = (NB, c["Hkv"], bs, c["D"]), (NB, c["Hkv"], c["D"], bs)
    if c["fmt"]:
        kc = synth.normal_codes_host(kshape, seed + 1, c["fmt"])
        vc = synth.normal_codes_host(vshape, seed + 2, c["fmt"])
    else:
        kc = synth.normal_host(kshape, seed + 1, c["dt"])
        vc = synth.normal_host(vshape, seed + 2, c["dt"])
    c.update(tables=tables, kc=kc, vc=vc, MB=MB, max_ctx=MB * bs)


def device_pools(c):
    if c["fmt"]:
        return torch.from_numpy(c["kc"]).cuda(), torch.from_numpy(c["vc"]).cuda()
    return synth.to_torch(c["kc"], c["dt"]).cuda(), synth.to_torch(c["vc"], c["dt"]).cuda()


@pytest.mark.parametrize("case", range(CASES))
def test_random_case_matches_the_oracle(case):
    run_case(case, 1.0)


@pytest.mark.parametrize("case", range(WIDE_CASES))
def test_random_case_with_wide_logits(case):
    run_case(case, WIDE_GAIN)


def run_case(case, gain):
    rng, c = draw(case)
    print(f"fuzz case {case} (scale x {gain}): "
          f"{dict((k, c[k]) for k in ('fmt', 'dt', 'D', 'bs', 'Hkv', 'H', 'S', 'ctx', 'path', 'ps'))}", flush=True)
    build(rng, c, 7000 + case)
    kc, vc = device_pools(c)
    tab = torch.from_numpy(c["tables"]).cuda()
    lens = torch.tensor(c["ctx"], dtype=torch.int32).cuda()
    quant = (c["fmt"], K_SCALE, V_SCALE) if c["fmt"] else None
    scale = float(np.float32(scale_for(c["D"]) * gain))
    split = c["path"].endswith("split")
    path = c["path"].split("-")[0]
    if path == "multi":
        spans = [int(rng.integers(0, min(n, 9) + 1)) for n in c["ctx"]]
        if sum(spans) == 0 and max(c["ctx"]) > 0:  # at least one query row
            spans[int(np.argmax(c["ctx"]))] = 1
        if sum(spans) == 0:                        # every context empty: plain decode instead
            path = "single"
    if path == "multi":
        qstart = np.concatenate([[0], np.cumsum(spans)]).astype(np.int32)
        T = int(qstart[-1])
        q = synth.normal_host((max(T, 1), c["H"], c["D"]), 7000 + case + 3, c["dt"])[:T]
        ref = A.paged_decode_multi(q, c["kc"], c["vc"], c["tables"], c["ctx"], qstart, scale, c["dt"], quant=quant)
        qd = synth.to_torch(q, c["dt"]).cuda()
        out = torch.full_like(qd, 7.0)
        ws = None
        if split:
            ws = torch.empty(pa.pa_decode_multi_workspace_bytes(T, c["H"], c["D"], c["max_ctx"], c["ps"]),
                             dtype=torch.uint8, device="cuda")
        pa.pa_decode_multi(out, qd, kc, vc, tab, lens, torch.from_numpy(qstart).cuda(), max(spans + [1]),
                           c["max_ctx"], scale, K_SCALE, V_SCALE, kv_format=c["fmt"], partition_size=c["ps"],
                           workspace=ws, split=split)
    else:
        q = synth.normal_host((c["S"], c["H"], c["D"]), 7000 + case + 3, c["dt"])
        qd = synth.to_torch(q, c["dt"]).cuda()
        out = torch.full_like(qd, 7.0)
        ws = None
        if split:
            ws = torch.empty(pa.pa_decode_split_workspace_bytes(c["S"], c["H"], c["D"], c["max_ctx"], c["ps"]),
                             dtype=torch.uint8, device="cuda")
        if path == "masked":
            lo, hi = [], []
            for n in c["ctx"]:
                a = int(rng.integers(0, n + 1))
                b = int(rng.integers(a, n + 1))
                lo.append(a)
                hi.append(b)
            ref = A.paged_decode(q, c["kc"], c["vc"], c["tables"], c["ctx"], scale, c["dt"], quant=quant,
                                 masks=(lo, hi))
            pa.pa_decode_masked(out, qd, kc, vc, tab, lens, torch.tensor(lo, dtype=torch.int32).cuda(),
                                torch.tensor(hi, dtype=torch.int32).cuda(), c["max_ctx"], scale, K_SCALE, V_SCALE,
                                kv_format=c["fmt"], partition_size=c["ps"], workspace=ws, split=split)
        else:
            ref = A.paged_decode(q, c["kc"], c["vc"], c["tables"], c["ctx"], scale, c["dt"], quant=quant)
            if c["fmt"]:
                pa.pa_decode_quant(out, qd, kc, vc, tab, lens, c["max_ctx"], scale, K_SCALE, V_SCALE,
                                   kv_format=c["fmt"], partition_size=c["ps"], workspace=ws, split=split)
            elif split:
                pa.pa_decode_split(out, qd, kc, vc, tab, lens, c["max_ctx"], scale, c["ps"], ws)
            else:
                pa.pa_decode(out, qd, kc, vc, tab, lens, c["max_ctx"], scale)
    torch.cuda.synchronize()
    extra = 0.0
    if gain != 1.0:
        extra = output_rounding_term(ref, c["dt"])
    if c["dt"] == "f32" and gain != 1.0:
        extra = extra + fp32_logit_term(max_abs_logit2(q, c["kc"], c["tables"], c["ctx"], c["bs"], "f32", scale),
                                float(np.max(np.abs(A.to_f64(c["vc"], "f32")))))
    assert_close(out_to_f64(out, c["dt"]), ref, c["dt"], f"fuzz case {case} x {gain} ({c['path']})", extra)
