"""Seeded random sessions of the PagedAttention object, every step against attention over
each request's tokens kept contiguous on the host.

A case draws a pool (fp32 / fp16 / bf16, or FP8 E4M3, int8 or row-scaled int8 codes under
fp16 / bf16 queries), head_dim, block size, KV heads and group size, then runs twelve steps.
Before each step one event is drawn: a new request (sometimes on one of two cached prompt
prefixes, stored once on a miss), a fork, a free, a swap out or back in, or a sliding
window.  Each step decodes a random subset of the requests on the device in random order
(forks are sometimes passed next to their parent), so the object takes every decode path
it has (pa_decode_auto / pa_decode_quant, pa_decode_shared, pa_decode_masked) and every
copy it makes (copy-on-write, swap).  A step that names a swapped request must fail
before it changes anything.  8-bit pools are compared with attention over the rows the
oracle's quantisation gives.  The draws come from numpy PCG64 seeded by the case number,
so a failing case is reproduced by its id."""
import numpy as np
import pytest
import torch

import paged_kv_cache_333_amd as pa
import synth
from oracle import attention as A
from tests.gpu_helpers import assert_close, out_to_f64
from tests.test_gpu_paged_attention import contiguous_reference, stored_rows

pytestmark = pytest.mark.gpu

CASES = 48
STEPS = 12
K_SCALE, V_SCALE = 0.04, 0.035
PREFIXES = {0: list(range(5000, 5020)), 1: list(range(6000, 6037))}   # cached prompt prefixes (token ids)


def draw(case):
    rng = np.random.default_rng(9100 + case)
    fmt = [None, None, "fp8_e4m3", "int8", "int8_token"][int(rng.integers(5))]
    dt = ["f16", "bf16"][int(rng.integers(2))] if fmt else ["f32", "f16", "bf16"][int(rng.integers(3))]
    D = int(rng.choice([64, 128]))
    sizes = [16, 32] + ([64] if D == 128 else []) + ([8] if D == 128 and not fmt else [])
    bs = int(rng.choice(sizes))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    return rng, dict(fmt=fmt, dt=dt, D=D, bs=bs, Hkv=Hkv, H=Hkv * G)


class Session:
    def __init__(self, rng, c):
        self.rng, self.c = rng, c
        self.NB = 4096 // c["bs"]
        self.m = pa.PagedAttention(c["H"], c["D"], block_size=c["bs"], num_blocks=self.NB, num_kv_heads=c["Hkv"],
                                   dtype=synth.torch_dtype(c["dt"]), num_host_blocks=self.NB // 2,
                                   kv_format=c["fmt"], k_scale=K_SCALE, v_scale=V_SCALE)
        self.rows = {}       # request -> (K rows, V rows) as float64 [Hkv, D] each, in position order
        self.window = {}     # request -> window length
        self.where = {}      # request -> "device" | "host"
        self.kind = {}       # request -> "plain" | "prefix"
        self.parent = {}     # fork -> its parent
        self.prefix_rows = {}
        self.next_id = 1
        self.seed = 9100 * 1000 + 17 * int(rng.integers(1000))

    def _rows(self, n):
        c = self.c
        k = synth.normal_host((n, c["Hkv"], c["D"]), self.seed, c["dt"])
        v = synth.normal_host((n, c["Hkv"], c["D"]), self.seed + 1, c["dt"])
        self.seed += 2
        if c["fmt"]:
            kq, vq = stored_rows(k, v, c["dt"], c["fmt"], K_SCALE, V_SCALE)
        else:
            kq, vq = A.to_f64(k, c["dt"]), A.to_f64(v, c["dt"])
        dev = (synth.to_torch(k, c["dt"]).cuda(), synth.to_torch(v, c["dt"]).cuda())
        return dev, (list(kq), list(vq))

    def on_device(self, pred=lambda r: True):
        return [r for r in self.rows if self.where[r] == "device" and pred(r)]

    # -- events ----------------------------------------------------------------
    def new_request(self):
        rng, bs = self.rng, self.c["bs"]
        r = self.next_id
        self.next_id += 1
        if rng.random() < 0.3:
            which = int(rng.integers(2))
            toks = PREFIXES[which]
            own = int(rng.integers(1, 2 * bs + 1))
            pid, hit, start = self.m.allocate_with_prefix(r, toks, own)
            if not hit:
                (pk, pv), self.prefix_rows[which] = self._rows(len(toks))
                self.m.store_prefix(pid, pk, pv)
            (k, v), (kq, vq) = self._rows(own)
            self.m.store(r, k, v, start=start)
            prk, prv = self.prefix_rows[which]
            self.rows[r] = (list(prk) + kq, list(prv) + vq)
            self.kind[r] = "prefix"
        else:
            n = int(rng.integers(1, 4 * bs + 6))
            self.m.allocate(r, n)
            (k, v), self.rows[r] = self._rows(n)
            self.m.store(r, k, v)
            self.kind[r] = "plain"
        self.where[r] = "device"
        return f"new {r} ({self.kind[r]}, {self.m.context_len(r)} positions)"

    def event(self):
        rng = self.rng
        plain = self.on_device(lambda r: self.kind[r] == "plain" and r not in self.window)
        choices = ["new"] * 2
        if plain:
            choices += ["fork"] * 2 + ["swap out"]
        if any(w == "host" for w in self.where.values()):
            choices += ["swap in"] * 2
        if len(self.rows) > 2:
            choices += ["free"]
        lonely = [r for r in plain if r not in self.parent and r not in self.parent.values()]
        if lonely:
            choices += ["window"]
        ev = choices[int(rng.integers(len(choices)))]
        if ev == "new" or not self.rows:
            return self.new_request()
        if ev == "fork":
            p = plain[int(rng.integers(len(plain)))]
            r = self.next_id
            self.next_id += 1
            self.m.fork(p, r)
            self.rows[r] = (list(self.rows[p][0]), list(self.rows[p][1]))
            self.where[r], self.kind[r], self.parent[r] = "device", "plain", p
            return f"fork {p} -> {r}"
        if ev == "swap out":
            r = plain[int(rng.integers(len(plain)))]
            self.m.swap_out([r])
            self.where[r] = "host"
            return f"swap out {r}"
        if ev == "swap in":
            host = [r for r, w in self.where.items() if w == "host"]
            r = host[int(rng.integers(len(host)))]
            self.m.swap_in([r])
            self.where[r] = "device"
            return f"swap in {r}"
        if ev == "free":
            ids = list(self.rows)
            r = ids[int(rng.integers(len(ids)))]
            self.m.free(r)
            for d in (self.rows, self.where, self.kind, self.window):
                d.pop(r, None)
            return f"free {r}"
        r = lonely[int(rng.integers(len(lonely)))]
        w = int(rng.integers(1, self.m.context_len(r) + 2))
        self.m.set_window(r, w)
        self.window[r] = w
        return f"window {r}: {w}"

    # -- one decode step ------------------------------------------------------------
    def step(self, k):
        rng, c = self.rng, self.c
        ids = self.on_device()
        if not ids:
            return "no request on the device"
        rng.shuffle(ids)
        ids = ids[:int(rng.integers(1, len(ids) + 1))]
        if rng.random() < 0.5:  # forks beside their parents
            ids.sort(key=lambda r: (self.parent.get(r, r), r))
        host = [r for r, w in self.where.items() if w == "host"]
        if host and rng.random() < 0.3:
            before = {r: self.m.context_len(r) for r in ids}
            with pytest.raises(pa.PAError):
                S = len(ids) + 1
                q = torch.zeros((S, c["H"], c["D"]), dtype=synth.torch_dtype(c["dt"]), device="cuda")
                kv = torch.zeros((S, c["Hkv"], c["D"]), dtype=q.dtype, device="cuda")
                self.m.forward(ids + [host[0]], q, kv, kv)
            assert {r: self.m.context_len(r) for r in ids} == before, "a refused step changed a length"
        S = len(ids)
        q = synth.normal_host((S, c["H"], c["D"]), self.seed, c["dt"])
        self.seed += 1
        (kn, vn), (kq, vq) = self._rows(S)
        out = self.m.forward(ids, synth.to_torch(q, c["dt"]).cuda(), kn, vn)
        torch.cuda.synchronize()
        for i, r in enumerate(ids):
            self.rows[r][0].append(kq[i])
            self.rows[r][1].append(vq[i])
        rows = [(self.rows[r][0][-self.window[r]:], self.rows[r][1][-self.window[r]:]) if r in self.window
                else self.rows[r] for r in ids]
        ref = contiguous_reference(q, rows, c["H"], c["Hkv"], self.m.scale, c["dt"], kv_f64=True)
        assert_close(out_to_f64(out, c["dt"]), ref, c["dt"], f"step {k}, requests {ids}, {self.m.last_path}")
        return f"step {k}: {ids} -> {self.m.last_path}"


@pytest.mark.parametrize("case", range(CASES))
def test_random_session_matches_contiguous_attention(case):
    rng, c = draw(case)
    print(f"object fuzz case {case}: {c}", flush=True)
    s = Session(rng, c)
    for _ in range(2):
        s.new_request()
    for k in range(STEPS):
        print("  " + s.event(), flush=True)
        print("  " + s.step(k), flush=True)
    for r in list(s.rows):
        s.m.free(r)
    assert s.m.allocator.num_free_blocks() == s.NB, "every block returns to the pool"
