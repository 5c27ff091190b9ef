"""Host-side arithmetic of bench.py, checked on the CPU: the number of decode steps a
workload's pool holds, against an allocator that actually appends the tokens."""
import bench
import synth
from oracle.allocator import AllocatorError, BlockAllocator


def grow_until_full(w, limit):
    alloc = BlockAllocator(w.num_blocks, w.block_size, [int(x) for x in w.free_order])
    for s, n in enumerate(w.context_lens):
        alloc.seq_create(s, n)
    for step in range(limit):
        try:
            for _ in range(w.query_len):
                alloc.seq_append_slots(list(range(w.num_seqs)))
        except AllocatorError:
            return step
    return limit


def test_steps_that_fit_matches_an_allocator_run():
    for key in (3, 7):  # the workloads whose pools are 1.1x their initial blocks
        w = synth.workload(key)
        fit = bench.steps_that_fit(w.context_lens, w.block_size, w.num_blocks, w.query_len, 400)
        assert 60 <= fit < 400  # the default 10 + 50 steps fit
        assert grow_until_full(w, 400) == fit


def test_steps_that_fit_caps_at_the_steps_asked_for():
    w = synth.workload(2)
    assert bench.steps_that_fit(w.context_lens, w.block_size, w.num_blocks, w.query_len, 60) == 60
    assert bench.steps_that_fit([15], 16, 1, 1, 5) == 1  # one more token opens a second block
    assert bench.steps_that_fit([16], 16, 1, 1, 5) == 0


def test_more_than_one_gpu_is_refused_with_a_message():
    """bench.py measures one GPU: any other --gpus exits with status 2 and says why, before
    touching the GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=root, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and "--gpus 2" in r.stderr
