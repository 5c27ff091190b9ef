"""GPU parity of the shared-prefix decode (pa_decode_shared): families of forked sequences
that share their leading blocks, read once per family with each member seeing its own
prefix, then each sequence's own tokens, merged.  Against the float64 oracle's plain decode
(the definition does not change) for every model dtype and both 8-bit formats, head groups
1 to 8, families of 1 to 17 members (more members than the 16 columns of a tile), members
whose context ends inside the shared blocks, long prefixes over several partitions, empty
sequences; groups from pa_shared_prefix_groups, hand-made shorter prefixes and members of
one group with different prefixes; a prefix beyond its member's context gives that
member NaN rows.  Unused rows of the pools are poisoned."""
import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_333_amd as pa
import synth
from oracle import attention as A
from tests.gpu_helpers import (DeviceWorkload, assert_close, fp32_logit_term, max_abs_logit2, out_to_f64,
                               output_rounding_term, scale_for)

pytestmark = pytest.mark.gpu

KINDS = [("f32", None), ("f16", None), ("bf16", None), ("f16", "fp8_e4m3"), ("bf16", "int8")]
# (element type, 8-bit format, head_dim, block size); 8-bit pools take no 8-token blocks (the host
# rejects them, tested on the CPU)
POOL_CASES = [(dt, fmt, D, bs) for D, bs in [(64, 16), (128, 32), (128, 16), (128, 8), (128, 64)]
              for dt, fmt in KINDS if not (fmt and bs == 8)]
POISON_CODE = {"fp8_e4m3": 0x7F, "int8": 0x80}

# (blocks shared by the family at block size 16, context length of each member in tokens)
FAMILIES = [
    (3, [48, 50, 60, 88, 48]),      # five branches, three shared blocks (at bs 16), own tails
    (0, [70]),                      # a loner
    (3, [20, 60, 90]),              # a member whose context ends inside the shared blocks
    (2, [32 + k for k in range(17)]),   # 17 members: more than one tile of columns
    (0, [0]),                       # an empty sequence
    (40, [645, 700, 740, 800]),     # a long prefix over several partitions
]


def make_case(seed, dt, fmt, H, Hkv, D, bs, families=FAMILIES):
    """Tables where each family's members share `shared` leading blocks (scaled to bs so the
    token counts keep their meaning at other block sizes, at least one block) and own the rest."""
    rng = np.random.default_rng(seed)
    rows, ctx = [], []
    nxt = 0
    scale_bs = 16 / bs
    for shared, lens in families:
        sh = max(1, int(round(shared * scale_bs))) if shared else 0
        base = list(range(nxt, nxt + sh))
        nxt += sh
        for n in lens:
            need = -(-n // bs)
            own = list(range(nxt, nxt + max(need - sh, 0)))
            nxt += len(own)
            rows.append((base + own)[:need])
            ctx.append(n)
    NB = nxt + 3
    perm = rng.permutation(NB)
    MB = max(len(r) for r in rows) + 1
    tables = -np.ones((len(rows), MB), dtype=np.int32)
    for s, r in enumerate(rows):
        tables[s, :len(r)] = perm[np.array(r, dtype=np.int64)] if r else []
    S = len(rows)
    if fmt:
        kc = synth.normal_codes_host((NB, Hkv, bs, D), seed + 1, fmt)
        vc = synth.normal_codes_host((NB, Hkv, D, bs), seed + 2, fmt)
    else:
        kc = synth.normal_host((NB, Hkv, bs, D), seed + 1, dt)
        vc = synth.normal_host((NB, Hkv, D, bs), seed + 2, dt)
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
    q = synth.normal_host((S, H, D), seed + 3, dt)
    ks, vs = (float(np.float32(1.1 / synth.CODE_SIGMA[fmt])), float(np.float32(0.9 / synth.CODE_SIGMA[fmt]))) \
        if fmt else (1.0, 1.0)
    return dict(q=q, kc=kc, vc=vc, tables=tables, ctx=ctx, NB=NB, MB=MB, dt=dt, fmt=fmt, S=S, H=H, Hkv=Hkv, D=D,
                bs=bs, ks=ks, vs=vs)


def dev(c):
    d = "cuda"
    if c["fmt"]:
        kc, vc = torch.from_numpy(c["kc"]).to(d), torch.from_numpy(c["vc"]).to(d)
    else:
        kc, vc = synth.to_torch(c["kc"], c["dt"]).to(d), synth.to_torch(c["vc"], c["dt"]).to(d)
    return dict(q=synth.to_torch(c["q"], c["dt"]).to(d), kc=kc, vc=vc, tab=torch.from_numpy(c["tables"]).to(d),
                ctx=torch.tensor(c["ctx"], dtype=torch.int32, device=d))


def run_shared(c, dv, groups, cached=False, scale=None):
    gs, pl, ng, mg = groups
    max_ctx = c["MB"] * c["bs"]
    ws = torch.empty(pa.pa_decode_shared_workspace_bytes(c["S"], c["H"], c["D"], max_ctx), dtype=torch.uint8,
                     device="cuda")
    c["ws"] = ws
    out = torch.full_like(dv["q"], 7.0)
    pa.pa_decode_shared(out, dv["q"], dv["kc"], dv["vc"], dv["tab"], dv["ctx"],
                        torch.tensor(gs, dtype=torch.int32, device="cuda"),
                        torch.tensor(pl, dtype=torch.int32, device="cuda"), ng, mg, max_ctx,
                        scale_for(c["D"]) if scale is None else scale, ws, c["ks"], c["vs"], kv_format=c["fmt"],
                        cached_kv=cached)
    torch.cuda.synchronize()
    return out_to_f64(out, c["dt"])


def oracle(c):
    quant = (c["fmt"], c["ks"], c["vs"]) if c["fmt"] else None
    return A.paged_decode(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], scale_for(c["D"]), c["dt"], quant=quant)


@pytest.mark.parametrize("dt,fmt,D,bs", POOL_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 2), (16, 2), (32, 2)])
def test_shared_prefix_families(dt, fmt, D, bs, H, Hkv):
    c = make_case(zlib.crc32(repr((dt, fmt, D, bs, H, Hkv)).encode()) % 10000, dt, fmt, H, Hkv, D, bs)
    groups = pa.pa_shared_prefix_groups(c["tables"].tolist(), c["ctx"], bs)
    assert groups[2] < c["S"] and groups[3] == 17      # the families were found
    dv = dev(c)
    ref = oracle(c)
    got = run_shared(c, dv, groups)
    assert_close(got, ref, dt, "shared prefix")
    assert np.array_equal(run_shared(c, dv, groups, cached=True), got)
    # every sequence a group of its own: plain decode through the same two passes
    S = c["S"]
    assert_close(run_shared(c, dv, (list(range(S + 1)), [0] * S, S, 1)), ref, dt, "groups of one")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_shorter_hand_made_prefixes(dt):
    """Any prefix up to the shared blocks is valid: one block, or a length inside a block."""
    c = make_case(77, dt, None, 8, 2, 128, 16)
    gs, pl, ng, mg = pa.pa_shared_prefix_groups(c["tables"].tolist(), c["ctx"], 16)
    dv = dev(c)
    ref = oracle(c)
    for cut in (16, 9, 1):
        pl2 = [min(p, cut) if p else 0 for p in pl]
        assert_close(run_shared(c, dv, (gs, pl2, ng, mg)), ref, dt, f"prefix cut to {cut}")


def test_members_with_different_prefixes():
    """A member's prefix may be any length its blocks share with its group's row: members of
    one group cut to 32 and to 5 tokens (the rest read from their own blocks) match the
    oracle; a prefix longer than the member's context gives that member NaN rows only."""
    c = make_case(5, "f16", None, 4, 4, 64, 16)
    gs, pl, ng, mg = pa.pa_shared_prefix_groups(c["tables"].tolist(), c["ctx"], 16)
    assert pl[:5] == [48, 48, 48, 88, 48]     # the family's row is its longest member, 88 tokens
    pl[1] = 32
    pl[2] = 5
    ref = oracle(c)
    got = run_shared(c, dev(c), (gs, pl, ng, mg))
    assert_close(got, ref, "f16", "different prefixes")
    pl[4] = 60                                   # beyond its 48 tokens
    got = run_shared(c, dev(c), (gs, pl, ng, mg))
    assert np.all(np.isnan(got[4]))
    ok = [s for s in range(c["S"]) if s != 4]
    assert_close(got[ok], ref[ok], "f16", "the other sequences")


def test_parallel_sampling_workload_full_size_every_row():
    """The parallel-sampling workload (32 parents of 2304 tokens, 5 branches each forked at
    2048-2304 tokens, fp16, 32 heads) in its post-fork state: groups from the allocator's
    tables, every output row against the oracle (the step with its copies and writes is
    test_gpu_bench_step.py's)."""
    dw = DeviceWorkload(5)
    w = dw.w
    tabs = dw.tables.cpu().tolist()
    lens = dw.context_lens.cpu().tolist()
    gs, pl, ng, mg = pa.pa_shared_prefix_groups(tabs, lens, w.block_size)
    assert ng == w.groups and mg == w.branches
    ws = torch.empty(pa.pa_decode_shared_workspace_bytes(w.num_seqs, w.num_heads, w.head_dim, dw.max_context_len),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dw.query)
    pa.pa_decode_shared(out, dw.query, dw.key_cache, dw.value_cache, dw.tables, dw.context_lens,
                        torch.tensor(gs, dtype=torch.int32, device="cuda"),
                        torch.tensor(pl, dtype=torch.int32, device="cuda"), ng, mg, dw.max_context_len, w.scale, ws,
                        cached_kv=True)
    plain = torch.empty_like(dw.query)
    pa.pa_decode(plain, dw.query, dw.key_cache, dw.value_cache, dw.tables, dw.context_lens, dw.max_context_len,
                 w.scale, cached_kv=True)
    torch.cuda.synchronize()
    got = out_to_f64(out, w.dtype)
    ref = dw.oracle_all()
    assert_close(got, ref, w.dtype, "workload 5 post-fork, shared-prefix decode, every row")
    assert_close(out_to_f64(plain, w.dtype), ref, w.dtype, "workload 5 post-fork, plain decode, every row")


def test_group_larger_than_max_group_size_gets_nan_rows():
    """max_group_size below a group's size: that group's rows are NaN (none stale), the
    other groups still match the oracle."""
    c = make_case(6, "f16", None, 4, 4, 64, 16)
    gs, pl, ng, mg = pa.pa_shared_prefix_groups(c["tables"].tolist(), c["ctx"], 16)
    assert mg == 17
    dv = dev(c)
    run_shared(c, dv, (gs, pl, ng, mg))              # a valid call first: the workspace holds its lengths
    got = run_shared(c, dv, (gs, pl, ng, 5))
    big = [g for g in range(ng) if gs[g + 1] - gs[g] == 17][0]
    rows = list(range(gs[big], gs[big + 1]))
    assert np.all(np.isnan(got[rows]))
    ref = oracle(c)
    ok = [s for s in range(c["S"]) if s not in rows]
    assert_close(got[ok], ref[ok], "f16", "the other groups")


@pytest.mark.parametrize("parts", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("dt,fmt", [("f16", None), ("bf16", "int8")], ids=lambda v: str(v))
def test_every_forced_partition_count(parts, dt, fmt, monkeypatch):
    """The prefix pass's flat launch packs the partition waves of several units into one
    workgroup: every count 1..8 (PA_SHARED_PARTS) gives the oracle's result, including counts
    that four waves per workgroup do not divide and the last workgroup's waves past the last
    unit; the prefix lengths sit at the documented end of the workspace for every count; and
    the automatic choice agrees with the oracle too."""
    c = make_case(4242 + parts, dt, fmt, 8, 2, 128, 16)
    groups = pa.pa_shared_prefix_groups(c["tables"].tolist(), c["ctx"], 16)
    dv = dev(c)
    ref = oracle(c)
    monkeypatch.setenv("PA_SHARED_PARTS", str(parts))
    got = run_shared(c, dv, groups)
    assert_close(got, ref, dt, f"{parts} partitions")
    # the prefix length each sequence's partials cover: one int32 per sequence at the end of
    # the workspace, wherever this call's partition count put the partials
    S = c["S"]
    assert c["ws"].numel() % 4 == 0
    assert c["ws"][-4 * S:].view(torch.int32).cpu().tolist() == list(groups[1])
    monkeypatch.delenv("PA_SHARED_PARTS")
    assert_close(run_shared(c, dv, groups), ref, dt, "automatic partition count")


RANDOM_CASES, WIDE_CASES, WIDE_GAIN = 48, 16, 40.0


def draw_families(case):
    """A random shared-prefix case: pool format, head shape, 1-5 families of 1-19 members
    sharing 0-29 leading blocks (counted at 16 tokens; make_case rescales them), members
    ending before, inside or after the shared blocks, and a forced partition count 1-8 or
    the automatic one (0)."""
    rng = np.random.default_rng(8800 + case)
    fmt = [None, None, "fp8_e4m3", "int8"][int(rng.integers(4))]
    dt = ["f16", "bf16"][int(rng.integers(2))] if fmt else ["f32", "f16", "bf16"][int(rng.integers(3))]
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32] + ([64] if D == 128 else []) + ([8] if D == 128 and not fmt else [])))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    fams = []
    for _ in range(int(rng.integers(1, 6))):
        shared = int(rng.integers(0, 30))
        lens = [int(rng.integers(max(0, 16 * shared - 24), 16 * shared + 120)) for _ in range(int(rng.integers(1, 20)))]
        fams.append((shared, lens))
    return dict(fmt=fmt, dt=dt, D=D, bs=bs, Hkv=Hkv, H=Hkv * G, fams=fams, parts=int(rng.integers(0, 9)))


def run_family_case(case, gain, monkeypatch):
    d = draw_families(case)
    print(f"shared-prefix case {case} (scale x {gain}): {d}", flush=True)
    c = make_case(8800 + case, d["dt"], d["fmt"], d["H"], d["Hkv"], d["D"], d["bs"], families=d["fams"])
    groups = pa.pa_shared_prefix_groups(c["tables"].tolist(), c["ctx"], c["bs"])
    scale = float(np.float32(scale_for(c["D"]) * gain))
    quant = (c["fmt"], c["ks"], c["vs"]) if c["fmt"] else None
    ref = A.paged_decode(c["q"], c["kc"], c["vc"], c["tables"], c["ctx"], scale, c["dt"], quant=quant)
    if d["parts"]:
        monkeypatch.setenv("PA_SHARED_PARTS", str(d["parts"]))
    got = run_shared(c, dev(c), groups, scale=scale)
    extra = 0.0 if gain == 1.0 else output_rounding_term(ref, c["dt"])
    if c["dt"] == "f32" and gain != 1.0:
        vals = A.to_f64(c["vc"], "f32")
        extra = extra + fp32_logit_term(max_abs_logit2(c["q"], c["kc"], c["tables"], c["ctx"], c["bs"], "f32", scale),
                                float(np.max(np.abs(vals[np.isfinite(vals)]))))
    assert_close(got, ref, c["dt"], f"shared-prefix case {case} x {gain}", extra)


@pytest.mark.parametrize("case", range(RANDOM_CASES))
def test_random_families_match_the_oracle(case, monkeypatch):
    """Seeded random shared-prefix cases (draw_families), every row against the oracle."""
    run_family_case(case, 1.0, monkeypatch)


@pytest.mark.parametrize("case", range(WIDE_CASES))
def test_random_families_with_wide_logits(case, monkeypatch):
    """The first random cases again with the softmax scale 40 times larger: the prefix
    partitions and the own tokens' partial then hold maxima hundreds apart, which the merge
    must rescale without overflow or loss."""
    run_family_case(case, WIDE_GAIN, monkeypatch)
