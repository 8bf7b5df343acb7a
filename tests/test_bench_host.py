"""CPU tests of bench.py's host logic: workload names (including the sweep families), the
algorithmic byte count, and the one-GPU guard."""
import subprocess
import sys

import numpy as np
import pytest

import bench
from workloads import synth


def test_sweep_workload_names():
    for n in (1, 7, 64):
        p = bench.workload_problem(f"decode7b_bs{n}")
        assert (p.n, p.h_in, p.h_out, p.r, p.dtype) == (n, 4096, 4096, 16, "f16")
        assert p.distinct_adapters() == n
    p = bench.workload_problem("prefill13b_down_len32")
    assert (p.n, p.h_in, p.h_out, p.dtype) == (128, 13824, 5120, "bf16")
    assert np.array_equal(np.unique(p.ids), np.arange(4))
    assert all(len(set(p.ids[32 * k: 32 * (k + 1)].tolist())) == 1 for k in range(4))
    for name in bench.SWEEPS["decode"] + bench.SWEEPS["prefill"]:
        bench.workload_problem(name)
    with pytest.raises(SystemExit):
        bench.workload_problem("decode7b_bs")


def test_algorithmic_bytes_by_hand():
    # 3 rows, two of them on adapter 1: x 3*8, y 2*3*4, A and B of 2 adapters 2*2*(8+4)
    p = synth.random_problem((9,), n=3, h_in=8, h_out=4, r=2, n_adapters=3, dtype="f16",
                             ids=np.array([1, 0, 1], np.int32))
    assert bench.algorithmic_bytes(p) == 2 * (3 * 8 + 2 * 3 * 4 + 2 * 2 * (8 + 4))
    assert bench.algorithmic_flops(p) == 2 * 3 * 2 * (8 + 4)


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, cwd=bench.ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_ranked_bytes_by_hand():
    # pools of ranks 16 (2 adapters) and 64 (1 adapter); rows on adapters 0, 2, 2
    q = synth.random_ranked_problem((9,), n=3, h_in=8, h_out=16, pools=[(2, 16), (1, 64)],
                                    dtype="bf16", ids=np.array([0, 2, 2], np.int32))
    assert bench.ranked_bytes(q) == 2 * (3 * 8 + 2 * 3 * 16 + (16 + 64) * (8 + 16))
    assert bench.ranked_flops(q) == 2 * (16 + 64 + 64) * (8 + 16)
    q = synth.mixed70b_ranked("k")
    assert q.n == 2112 and sorted(q.scales) == [16, 64]
    assert set(q.ranks()[q.ids[64:1088]]) == {16} and set(q.ranks()[q.ids[1088:]]) == {64}
