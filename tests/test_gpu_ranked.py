"""GPU tests of the mixed-rank call (sgmv_build_segments_ranked + sgmv_lora_add_ranked):
parity with the fp64 oracle, bit equality with one sgmv_lora_add per rank on that rank's
rows, the 70B mixed batch with ranks 16 and 64 at full size (every row) and HIP graph
replay."""
import sys

import numpy as np
import pytest

import oracle
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _assert_close(got, ref, what):
    err = np.abs(got - ref)
    tol = 1e-2 + 1e-2 * np.abs(ref)
    _say(f"{what}: max|err| {err.max():.3e}, worst err/tol {np.max(err / tol):.3f}")
    assert np.all(err <= tol), f"{what}: {int((err > tol).sum())} outside tolerance"


class Dev:
    """Device copies of a RankedProblem and its ranked batch."""

    def __init__(self, q):
        import torch
        from adapter_gemv_amd import sgmv
        self.q = q
        self.x = sgmv.as_tensor(q.x, q.dtype, "cuda")
        self.y0 = sgmv.as_tensor(q.y, q.dtype, "cuda")
        self.pools = [(sgmv.as_tensor(A, q.dtype, "cuda"), sgmv.as_tensor(B, q.dtype, "cuda"))
                      for A, B in q.pools]
        self.batch = sgmv.RankedBatch.build(q.ids, self.pools)
        torch.cuda.synchronize()

    def run(self, y=None, workspace=None):
        from adapter_gemv_amd import sgmv
        y = self.y0.clone() if y is None else y
        sgmv.lora_add_ranked(y, self.x, self.batch, self.q.scales, workspace)
        return y


def _storage(y, dtype):
    from adapter_gemv_amd.device_problem import to_numpy_storage
    return to_numpy_storage(y, dtype)


def _mixed70b_small():
    orig = synth.mixed70b_ids(np.random.default_rng(31))
    ids = np.where(orig % 2 == 0, orig // 2, 25 + orig // 2).astype(np.int32)
    return synth.random_ranked_problem((32, 1), n=ids.size, h_in=1024, h_out=1160,
                                       pools=[(25, 16), (25, 64)], dtype="bf16", ids=ids,
                                       name="mixed70b_small")


CASES = {
    "three_ranks_bf16": lambda: synth.random_ranked_problem(
        (30, 1), n=300, h_in=1032, h_out=776, pools=[(5, 16), (4, 32), (3, 64)], dtype="bf16"),
    "three_ranks_f16": lambda: synth.random_ranked_problem(
        (30, 2), n=97, h_in=520, h_out=1160, pools=[(9, 16), (2, 32), (7, 64)], dtype="f16"),
    "blocks_long": lambda: synth.random_ranked_problem(
        (30, 3), n=1100, h_in=2048, h_out=1032, pools=[(2, 16), (2, 64)], dtype="bf16",
        ids=np.repeat(np.random.default_rng(33).permutation(4), 275).astype(np.int32)),
    "one_row": lambda: synth.random_ranked_problem(
        (30, 4), n=1, h_in=4096, h_out=4096, pools=[(3, 16), (2, 64)], dtype="f16",
        ids=np.array([4], np.int32)),
    "one_rank_present": lambda: synth.random_ranked_problem(
        (30, 5), n=50, h_in=264, h_out=136, pools=[(3, 16), (3, 64)], dtype="bf16",
        ids=np.random.default_rng(34).integers(3, 6, 50).astype(np.int32)),
    "mixed70b_small": _mixed70b_small,
}


@pytest.mark.parametrize("name", list(CASES))
def test_ranked_parity(torch_cuda, name):
    q = CASES[name]()
    _say(f"[ranked] {name} n={q.n} h_in={q.h_in} h_out={q.h_out} ranks={sorted(q.scales)}")
    d = Dev(q)
    y = d.run()
    torch_cuda.cuda.synchronize()
    ref = oracle.lora_add_ranked(q.y, q.x, q.ids, q.pools, q.scales, q.dtype)
    _assert_close(oracle.decode(_storage(y, q.dtype), q.dtype), ref, name)


@pytest.mark.parametrize("name", ["three_ranks_bf16", "blocks_long", "mixed70b_small"])
def test_ranked_equals_one_call_per_rank(torch_cuda, name):
    """Each rank group runs the same kernels on the same sorted rows as sgmv_lora_add on
    that rank's rows alone, so the results agree bit for bit."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    q = CASES[name]()
    d = Dev(q)
    y = d.run()
    want = d.y0.clone()
    off = 0
    for (A, B), (A_h, _) in zip(d.pools, q.pools):
        P, r = A_h.shape[0], A_h.shape[1]
        rows = np.nonzero((q.ids >= off) & (q.ids < off + P))[0]
        if rows.size:
            _say(f"[ranked vs per-rank] {name} r={r} rows={rows.size}")
            idx = torch.as_tensor(rows, device="cuda")
            xs, ys = d.x[idx].contiguous(), want[idx].contiguous()
            b = sgmv.Batch.build(q.ids[rows] - off, A, B)
            sgmv.lora_add(ys, xs, b, q.scales[r])
            want[idx] = ys
        off += P
    torch.cuda.synchronize()
    assert torch.equal(y, want)


@pytest.mark.parametrize("proj", list(synth.MIXED70B_SHAPES))
def test_ranked_mixed70b_full_size(torch_cuda, proj):
    """The 70B mixed batch with ranks 16 and 64 in one call, at full size: all 2112 rows
    and every column against the oracle (evaluated in blocks of rows), eagerly and
    replayed from a HIP graph (the rank groups' chains side by side)."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    from parity_util import compare_all_rows
    q = synth.mixed70b_ranked(proj)
    _say(f"[ranked full] {q.name} n={q.n} h_in={q.h_in} h_out={q.h_out}")
    d = Dev(q)
    y = d.run()
    ws = sgmv.make_workspace(q.n, q.h_in, 64, torch.device("cuda"))
    yg = d.y0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d.run(yg, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.run(yg, ws)
    yg.copy_(d.y0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    outs = {"eager": _storage(y, q.dtype), "graph": _storage(yg, q.dtype)}
    del y, yg, g
    compare_all_rows(outs, q.n, lambda rows: oracle.lora_add_ranked(
        q.y[rows], q.x[rows], q.ids[rows], q.pools, q.scales, q.dtype), q.dtype, q.name)


def test_ranked_graph_replay(torch_cuda):
    """The ranked call captured in a HIP graph: every replay from the same y equals the
    eager result, with eager work and synchronisations between replays."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    q = CASES["three_ranks_bf16"]()
    d = Dev(q)
    eager = d.run()
    ws = sgmv.make_workspace(q.n, q.h_in, 64, torch.device("cuda"))
    y = d.y0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d.run(y, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.run(y, ws)
    for rep in range(3):
        y.copy_(d.y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[ranked graph] replay {rep}")
        assert torch.equal(y, eager)
        d.run()
        torch.cuda.synchronize()
