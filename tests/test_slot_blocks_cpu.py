"""The host check that picks pa_upload_and_cache's write form: a call's new tokens each
in a block of their own (slots outside [0, num_blocks * block_size) are skipped, as the
write skips them).  Both of its paths, the per-block stamp array and the sort used for
pools above the stamp bound or with more than 16 blocks per token of the call, are compiled into a small CPU harness with g++ and compared
with a set-based count on seeded random calls that share one thread, as successive
library calls do (stamp reuse, pools that grow and shrink between calls)."""
import pathlib
import shutil
import subprocess

import numpy as np
import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
HARNESS = ROOT / "tests" / "csrc" / "slot_blocks_check.cpp"
INCLUDE = ROOT / "paged_kv_cache_333_amd" / "csrc"


def expected(slots, num_blocks, block_size):
    seen = set()
    for s in slots:
        if 0 <= s < num_blocks * block_size:
            b = s // block_size
            if b in seen:
                return 0
            seen.add(b)
    return 1


def make_cases(seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(3000):
        bs = int(rng.choice([1, 16, 32]))
        nb = int(rng.integers(1, 400))
        n = int(rng.integers(0, 48))
        kind = i % 5
        if kind == 0:  # distinct blocks, a random offset in each: always 1
            blocks = rng.permutation(nb)[: min(n, nb)]
            slots = [int(b) * bs + int(rng.integers(0, bs)) for b in blocks]
        elif kind == 1:  # consecutive tokens of a few sequences (several per block when bs > 1)
            starts = rng.integers(0, nb * bs, size=max(1, n // 4))
            slots = [int(s) + j for s in starts for j in range(4) if int(s) + j < nb * bs]
        elif kind == 2:  # skipped slots mixed in: negative, past the pool
            slots = [int(x) for x in rng.integers(-3, nb * bs + 3 * bs, size=n)]
        elif kind == 3:  # two tokens at the two ends of one block
            b = int(rng.integers(0, nb))
            slots = [b * bs, b * bs + bs - 1] + [int(x) for x in rng.integers(0, nb * bs, size=n // 8)]
        else:  # skipped slots repeated right at the bounds, around the last block's own token
            slots = [nb * bs, -1, nb * bs, -1, nb * bs - 1]
        limit = nb if rng.random() < 0.5 else 0  # 0: the sort path
        cases.append((nb, bs, limit, slots))
    return cases


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_both_paths_match_a_set_count(tmp_path):
    exe = tmp_path / "slot_blocks_check"
    subprocess.run(["g++", "-O1", "-std=c++17", f"-I{INCLUDE}", str(HARNESS), "-o", str(exe)], check=True)
    cases = make_cases(7)
    text = [str(len(cases))]
    for nb, bs, limit, slots in cases:
        text.append(" ".join(map(str, [nb, bs, limit, len(slots), *slots])))
    out = subprocess.run([str(exe)], input="\n".join(text) + "\n", capture_output=True, text=True, check=True)
    got = [int(x) for x in out.stdout.split()]
    want = [expected(slots, nb, bs) for nb, bs, _, slots in cases]
    assert len(got) == len(cases)
    bad = [i for i, (g, w) in enumerate(zip(got, want)) if g != w]
    assert not bad, f"{len(bad)} mismatches, first case {cases[bad[0]][:3]}"
    assert 0 < sum(want) < len(want)  # both answers occur
