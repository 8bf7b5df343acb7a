"""GPU parity of libsgmv against the fp64 oracle, through the C ABI.

Tolerance (fp16/bf16 I/O, float32 accumulation): |y_gpu - y_ref| <= 1e-2 + 1e-2 |y_ref|
elementwise, y_ref being the unrounded fp64 oracle.  Segment gathering and exact-grid
inputs are checked bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
from workloads import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-2
RTOL = 1e-2


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _upload(p, **kw):
    from adapter_gemv_amd.device_problem import DeviceProblem
    return DeviceProblem.upload(p, **kw)


def _y_f64(y, dtype):
    from adapter_gemv_amd.device_problem import to_numpy_storage
    return oracle.decode(to_numpy_storage(y, dtype), dtype)


def _assert_close(got, ref, what):
    err = np.abs(got - ref)
    tol = ATOL + RTOL * np.abs(ref)
    bad = err > tol
    _say(f"{what}: max|err| {err.max():.3e}, worst err/tol {np.max(err / tol):.3f}")
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance"


def _run_lora(p, **kw):
    import torch
    dp = _upload(p, **kw)
    y = dp.lora_add()
    torch.cuda.synchronize()
    return dp, y


# --------------------------------------------------------------------------------------
# the workloads at full size
# --------------------------------------------------------------------------------------
SMALL = ["tiny", "decode7b", "sweep_a", "sweep_b", "sweep_c",
         "prefill13b_qo", "prefill13b_gateup", "prefill13b_down"]
FACT = dict(synth.all_workloads())


@pytest.mark.parametrize("name", SMALL)
def test_workload_full_compare(torch_cuda, name):
    _say(f"[parity] {name}")
    p = FACT[name]()
    _, y = _run_lora(p)
    _assert_close(_y_f64(y, p.dtype), oracle.lora_add_problem(p), name)


MIXED = [f"mixed70b_r{r}_{proj}" for r in (16, 64) for proj in synth.MIXED70B_SHAPES]


@pytest.mark.parametrize("name", MIXED)
def test_mixed70b_all_rows(torch_cuda, name):
    """The full 70B mixed batch (2112 rows, every column) in the benchmark's launch
    configuration, through host segment tables (sgmv_lora_add) and through device ids
    (sgmv_lora_add_pool: device grouping + the same table kernels), both against the
    oracle evaluated in blocks of rows (rows are independent)."""
    from adapter_gemv_amd.device_problem import to_numpy_storage
    from parity_util import compare_all_rows
    _say(f"[parity] {name}")
    p = FACT[name]()
    dp, y_tab = _run_lora(p)
    y_dev = dp.lora_add_pool()
    torch_cuda.cuda.synchronize()
    outs = {"host tables": to_numpy_storage(y_tab, p.dtype),
            "device ids": to_numpy_storage(y_dev, p.dtype)}
    del y_tab, y_dev, dp
    compare_all_rows(outs, p.n, lambda rows: oracle.lora_add(p.y[rows], p.x[rows], p.ids[rows],
                                                             p.A, p.B, p.scale, p.dtype),
                     p.dtype, name)


# --------------------------------------------------------------------------------------
# bit-exact: power-of-two grids and gather probes
# --------------------------------------------------------------------------------------
EXACT_CASES = [
    # name, n, h_in, h_out, r, P, ids-kind
    ("decode", 40, 4096, 4096, 16, 40, "perm"),
    ("short_mixed", 61, 1032, 520, 16, 9, "uniform"),
    ("long_only", 96, 2048, 1024, 16, 3, "blocks"),
    ("mixed_long_short", 150, 520, 1048, 32, 6, "mixed"),
    ("r64_mixed", 90, 1024, 776, 64, 5, "mixed"),
    ("r64_decode", 12, 8192, 1024, 64, 12, "perm"),
    ("deep_k", 40, 28672, 264, 16, 3, "mixed"),
    ("deep_k_long", 150, 20480, 264, 16, 3, "mixed"),  # r = 16 with 64-row shrink tiles
    # r = 16, short and long segments, 6144 < h_in <= 16384: the LDS-staged shrink with a
    # reduce pass, ragged last tile
    ("lds_r16_mixed", 150, 8200, 1032, 16, 12, "mixed"),
    # long segments only, 1100 rows (a ragged last tile of three-pass expand tiles)
    ("long_1100", 1100, 1032, 1048, 16, 3, "blocks"),
]


def _ids(kind, n, P, rng):
    if kind == "mixed70b":
        return synth.mixed70b_ids(rng)
    if kind == "perm":
        return rng.permutation(n).astype(np.int32) % P
    if kind == "uniform":
        return rng.integers(0, P, n).astype(np.int32)
    if kind == "blocks":
        return np.repeat(rng.permutation(P), -(-n // P))[:n].astype(np.int32)
    # a few long segments plus scattered short ones
    ids = rng.integers(2, P, n).astype(np.int32)
    ids[rng.choice(n, n // 3, replace=False)] = 0
    ids[rng.choice(n, n // 4, replace=False)] = 1
    return ids


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", EXACT_CASES, ids=[c[0] for c in EXACT_CASES])
def test_exact_grid_bit_exact(torch_cuda, case, dtype):
    name, n, h_in, h_out, r, P, kind = case
    _say(f"[exact] {name} {dtype}")
    rng = np.random.default_rng(sum(map(ord, name)))
    p = synth.exact_problem((31, len(name)), n=n, h_in=h_in, h_out=h_out, r=r, n_adapters=P,
                            dtype=dtype, ids=_ids(kind, n, P, rng))
    _, y = _run_lora(p)
    from adapter_gemv_amd.device_problem import to_numpy_storage
    got = to_numpy_storage(y, dtype).view(np.uint16)
    want = oracle.round_io(oracle.lora_add_problem(p), dtype).view(np.uint16)
    mism = got != want
    assert not mism.any(), f"{int(mism.sum())} elements differ"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("r,kind,n", [(16, "perm", 24), (16, "mixed", 120), (64, "mixed", 100),
                                      (32, "uniform", 57), (32, "mixed", 130)])
def test_gather_probe_bit_exact(torch_cuda, dtype, r, kind, n):
    _say(f"[gather] r={r} {kind} n={n} {dtype}")
    P = 6
    rng = np.random.default_rng(r + n)
    p = synth.gather_probe((41, r, n), n=n, h_in=512, h_out=384, r=r, n_adapters=P, dtype=dtype,
                           ids=_ids(kind, n, P, rng))
    _, y = _run_lora(p)
    from adapter_gemv_amd.device_problem import to_numpy_storage
    got = to_numpy_storage(y, dtype).view(np.uint16)
    want = oracle.round_io(oracle.lora_add_problem(p), dtype).view(np.uint16)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------------------
# ragged sizes, strides, edge cases
# --------------------------------------------------------------------------------------
RAGGED = [
    # n, h_in, h_out, r, P, ids-kind, ld_pad, identity_perm
    (1, 8, 8, 16, 1, "uniform", 0, False),
    (37, 200, 136, 16, 5, "uniform", 8, False),
    (15, 4104, 2056, 16, 1, "blocks", 0, True),     # longest short segment
    (16, 4104, 2056, 16, 1, "blocks", 0, True),     # shortest long segment
    (17, 1000, 3000, 32, 2, "blocks", 16, False),
    (333, 776, 1304, 64, 7, "mixed", 0, False),
    (257, 5128, 520, 16, 3, "mixed", 24, False),
    (64, 24, 4104, 64, 64, "perm", 0, False),
    (2048, 264, 264, 16, 1, "blocks", 0, True),     # one very long segment
    (300, 1032, 1160, 32, 3, "mixed", 8, False),    # r = 32 tiles, ragged last strip
    (129, 2056, 200, 64, 2, "blocks", 0, False),    # r = 64 tiles, narrow h_out
    (130, 16392, 1032, 16, 3, "mixed", 8, False),   # r = 16, 64-row shrink tiles, ragged
    (80, 264, 136, 64, 2, "blocks", 0, False),      # r = 64 LDS-staged shrink: one chunk,
                                                    # v written directly, padded stages
    (70, 16648, 520, 16, 2, "blocks", 8, False),    # r = 16 LDS-staged shrink, last chunk
                                                    # padded to a whole ring turn
    (150, 8200, 1032, 16, 12, "mixed", 8, False),   # r = 16 LDS-staged shrink at
                                                    # 6144 < h_in <= 16384 (short segments
                                                    # present), ragged last tile
    (2112, 8192, 1024, 16, 50, "mixed70b", 0, False),  # the 70B k/v shape at full size
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("case", RAGGED, ids=[f"n{c[0]}_{c[1]}x{c[2]}_r{c[3]}" for c in RAGGED])
def test_ragged_and_strided(torch_cuda, case, dtype):
    n, h_in, h_out, r, P, kind, ld_pad, ident = case
    _say(f"[ragged] {case} {dtype}")
    rng = np.random.default_rng(n * 7 + h_in)
    ids = _ids(kind, n, P, rng)
    if ident:
        ids = np.sort(ids)
    p = synth.random_problem((51, n, h_in, h_out, r), n=n, h_in=h_in, h_out=h_out, r=r,
                             n_adapters=P, dtype=dtype, ids=ids, scale=0.75)
    _, y = _run_lora(p, ld_pad=ld_pad, identity_perm=ident)
    _assert_close(_y_f64(y, dtype), oracle.lora_add_problem(p), f"ragged {case} {dtype}")


@pytest.mark.parametrize("r", [16, 64])
def test_fp16_long_segments_beyond_fp16_range(torch_cuda, r):
    """scale * v far beyond fp16's largest value (about 1.3e5 here) while every update fits
    in fp16: the long-segment expand feeds scale * v to MFMA as fp16 halves, so it must
    bring each row into range first; the GEMV rows of the same call check the other path."""
    import dataclasses
    _say(f"[fp16 range] r={r}")
    ids = np.concatenate([np.repeat([0, 1], 48), np.arange(2, 7)]).astype(np.int32)
    p = synth.random_problem((62, r), n=ids.size, h_in=256, h_out=648, r=r, n_adapters=7,
                             dtype="f16", ids=ids, scale=64.0)
    A = synth.quantize(p.A.astype(np.float32) * 2000.0, "f16")
    B = synth.quantize(p.B.astype(np.float32) / 2000.0, "f16")
    p = dataclasses.replace(p, A=A, B=B)
    v = np.einsum("nk,njk->nj", p.x.astype(np.float64), A.astype(np.float64)[p.ids])
    assert np.abs(p.scale * v).max() > 65504.0 * 1.5
    _, y = _run_lora(p)
    got = _y_f64(y, "f16")
    assert np.isfinite(got).all()
    _assert_close(got, oracle.lora_add_problem(p), f"fp16 range r={r}")


# --------------------------------------------------------------------------------------
# shrink and expand on their own
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("r,kind,n", [(16, "mixed", 200), (64, "mixed", 150), (32, "perm", 32)])
def test_shrink_and_expand(torch_cuda, dtype, r, kind, n):
    torch = torch_cuda
    _say(f"[shrink/expand] r={r} {kind} n={n} {dtype}")
    P = 8 if kind != "perm" else n
    rng = np.random.default_rng(3 * n + r)
    p = synth.random_problem((61, r, n), n=n, h_in=1544, h_out=1032, r=r, n_adapters=P,
                             dtype=dtype, ids=_ids(kind, n, P, rng))
    dp = _upload(p)
    v = dp.shrink()
    torch.cuda.synchronize()
    perm = dp.batch.table.perm
    v_ref = oracle.shrink(p.x, p.ids, p.A, dtype)[perm]          # sorted order
    _assert_close(v.double().cpu().numpy(), v_ref, "shrink v")
    # expand from the oracle's v (rounded to float32), in sorted order
    v_in = torch.as_tensor(v_ref.astype(np.float32), device=dp.x.device)
    y = dp.expand(v_in)
    torch.cuda.synchronize()
    y_ref = oracle.expand(p.y[perm], v_ref.astype(np.float32).astype(np.float64), p.ids[perm],
                          p.B, p.scale, dtype)
    _assert_close(_y_f64(y, dtype)[perm], y_ref, "expand y")


# --------------------------------------------------------------------------------------
# invariants on the GPU results
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_B_and_zero_scale_leave_y_unchanged(torch_cuda, dtype):
    _say(f"[invariant] zero B / zero scale {dtype}")
    rng = np.random.default_rng(5)
    p = synth.random_problem((71,), n=120, h_in=1032, h_out=776, r=16, n_adapters=5,
                             dtype=dtype, ids=_ids("mixed", 120, 5, rng))
    y0 = oracle.decode(p.y, dtype)
    dp = _upload(p)
    y = dp.lora_add(scale=0.0)
    torch_cuda.cuda.synchronize()
    assert np.array_equal(_y_f64(y, dtype), y0)
    p.B = np.zeros_like(p.B)
    dp = _upload(p)
    y = dp.lora_add()
    torch_cuda.cuda.synchronize()
    assert np.array_equal(_y_f64(y, dtype), y0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_shrink_linear_in_x_exactly(torch_cuda, dtype):
    _say(f"[invariant] v(2x) == 2 v(x) {dtype}")
    rng = np.random.default_rng(6)
    p = synth.random_problem((72,), n=140, h_in=2056, h_out=264, r=16, n_adapters=4,
                             dtype=dtype, ids=_ids("mixed", 140, 4, rng))
    v1 = _upload(p).shrink()
    p.x = synth.quantize(oracle.decode(p.x, dtype) * 2, dtype)
    v2 = _upload(p).shrink()
    torch_cuda.cuda.synchronize()
    assert torch_cuda.equal(v2, 2 * v1)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_row_order_independence(torch_cuda, dtype):
    """Permuting the caller's rows permutes the output (bit for bit: each row's sums do
    not depend on its position)."""
    _say(f"[invariant] row order {dtype}")
    rng = np.random.default_rng(8)
    p = synth.random_problem((73,), n=180, h_in=1032, h_out=520, r=16, n_adapters=6,
                             dtype=dtype, ids=_ids("mixed", 180, 6, rng))
    _, y1 = _run_lora(p)
    q = rng.permutation(p.n)
    p2 = synth.Problem("perm", dtype, p.ids[q], p.x[q], p.y[q], p.A, p.B, p.scale)
    _, y2 = _run_lora(p2)
    assert torch_cuda.equal(y2, y1[torch_cuda.as_tensor(q, device=y1.device)])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_identical_adapter_equals_any_split(torch_cuda, dtype):
    _say(f"[invariant] split adapter {dtype}")
    n = 64
    p = synth.random_problem((74,), n=n, h_in=2056, h_out=1032, r=16, n_adapters=1,
                             dtype=dtype, ids=np.zeros(n, np.int32))
    _, y1 = _run_lora(p)
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 5, n).astype(np.int32)
    p2 = synth.Problem("split", dtype, ids, p.x, p.y, np.repeat(p.A, 5, 0), np.repeat(p.B, 5, 0),
                       p.scale)
    _, y2 = _run_lora(p2)
    a, b = _y_f64(y1, dtype), _y_f64(y2, dtype)
    _assert_close(b, a, "split vs identical")
    _assert_close(a, oracle.lora_add_problem(p), "identical vs oracle")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_deterministic_and_workspace_reuse(torch_cuda, dtype):
    torch = torch_cuda
    _say(f"[determinism] {dtype}")
    from adapter_gemv_amd import sgmv
    rng = np.random.default_rng(10)
    p = synth.random_problem((75,), n=300, h_in=4096, h_out=2048, r=16, n_adapters=9,
                             dtype=dtype, ids=_ids("mixed", 300, 9, rng))
    dp = _upload(p)
    ws = sgmv.make_workspace(p.n, p.h_in, 16, dp.x.device)
    outs = [dp.lora_add(workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


# --------------------------------------------------------------------------------------
# the LoRA linear layer end to end (backbone GEMM + SGMV on one stream, graph-captured)
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["decode7b", "tiny"])
def test_lora_layer_end_to_end(torch_cuda, name):
    import bench
    _say(f"[layer] {name}")
    p = FACT[name]() if name in FACT else bench.workload_problem(name)
    r = bench.layer_measure(p, torch_cuda.device("cuda:0"), 8)
    _say(f"[layer] {name}: {r}")
    assert r["parity"]["ok"], r["parity"]
    assert r["layer_us"] > 0 and r["backbone_us"] > 0


def test_lora_layer_table_path(torch_cuda):
    """A prefill-sized layer through the table path (segment tables uploaded before
    graph capture)."""
    import bench
    _say("[layer] table path")
    p = synth.random_problem((91,), n=300, h_in=1032, h_out=776, r=16, n_adapters=3,
                             dtype="bf16", id_dist="uniform")
    r = bench.layer_measure(p, torch_cuda.device("cuda:0"), 8)
    _say(f"[layer] table: {r}")
    assert r["path"].startswith("table")
    assert r["parity"]["ok"], r["parity"]


# --------------------------------------------------------------------------------------
# short and long segments in one call: eager (one stream) against graph replay (the short
# chain on a forked second stream), bit for bit
# --------------------------------------------------------------------------------------
def _mixed_ids(n_long, n_short_each, n_short_adapters, seed):
    """Two long segments (adapters 0 and 1) and short segments on adapters 2 .., interleaved
    in caller order."""
    rng = np.random.default_rng(seed)
    ids = np.concatenate([np.zeros(n_long, np.int32), np.ones(n_long, np.int32),
                          np.repeat(np.arange(2, 2 + n_short_adapters, dtype=np.int32), n_short_each)])
    return rng.permutation(ids).astype(np.int32)


# (r, h_in, h_out, long rows per segment, short rows per segment, short segments):
#   r = 16, h_in = 8200: 17 GEMV slices and the LDS-staged shrink's many slices, each
#   kind summed by its own reduce pass;
#   r = 32: few GEMV slices summed by the GEMV expand, the long rows' few slices by the
#   MFMA expand; r = 64: reduce passes on both sides
GRAPH_MIXED = [(16, 8200, 1032, 520, 3, 9), (32, 1032, 2056, 40, 5, 4), (64, 2056, 1032, 70, 15, 3)]


@pytest.mark.parametrize("r,h_in,h_out,n_long,n_short,n_sa", GRAPH_MIXED)
def test_mixed_batch_graph_equals_eager(torch_cuda, r, h_in, h_out, n_long, n_short, n_sa):
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    _say(f"[graph mixed] r={r} h_in={h_in} h_out={h_out}")
    ids = _mixed_ids(n_long, n_short, n_sa, 7 + r)
    p = synth.random_problem((93, r), n=len(ids), h_in=h_in, h_out=h_out, r=r,
                             n_adapters=2 + n_sa, dtype="bf16", ids=ids)
    dp = _upload(p)
    ws = sgmv.make_workspace(p.n, p.h_in, r, dp.x.device)
    y_eager = dp.lora_add(workspace=ws)
    torch.cuda.synchronize()
    # every row and column of the eager call against the oracle
    _assert_close(_y_f64(y_eager, p.dtype), oracle.lora_add_problem(p), f"mixed r={r} eager")
    y = dp.fresh_y()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dp.lora_add(y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.lora_add(y, workspace=ws)
    for rep in range(3):
        y.copy_(dp.y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[graph mixed] r={r} replay {rep}")
        assert torch.equal(y, y_eager), f"replay {rep} differs from the eager call"
        _ = (dp.x.float() * 2).sum()
        torch.cuda.synchronize()


# (r, h_in, h_out): both reduce passes of a mixed call (r = 16 with the LDS-staged shrink,
# r = 64), and r = 32 (GEMV slices summed by the GEMV expand, long slices by the MFMA
# expand)
FLIP = [(16, 8200, 1032), (32, 1032, 2056), (64, 2056, 1032)]


@pytest.mark.parametrize("r,h_in,h_out", FLIP)
def test_graph_calls_whose_segments_change_kind(torch_cuda, r, h_in, h_out):
    """Two calls captured in one graph on one workspace, with different ids: the rows at
    the start of the sorted order belong to a 40-row (long) segment in the first call and
    to a 5-row (short) one in the second, and the reverse for a later segment.  Under
    capture each call's short and long chains run side by side; every slice count the
    reduce passes read must be the current call's.  Every replay must equal the eager
    calls bit for bit (eager: fresh workspaces)."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    _say(f"[graph flip] r={r} h_in={h_in} h_out={h_out}")
    rng = np.random.default_rng(500 + r)
    short = np.repeat(np.arange(2, 10, dtype=np.int32), 3)
    ids1 = rng.permutation(np.concatenate([np.zeros(40, np.int32), np.ones(5, np.int32), short]))
    ids2 = rng.permutation(np.concatenate([np.zeros(5, np.int32), np.ones(40, np.int32), short]))
    n = ids1.size
    assert ids2.size == n
    p = synth.random_problem((94, r), n=n, h_in=h_in, h_out=h_out, r=r, n_adapters=10,
                             dtype="bf16", ids=ids1)
    dp = _upload(p)
    b1 = sgmv.Batch.build(ids1, dp.A, dp.B)
    b2 = sgmv.Batch.build(ids2, dp.A, dp.B)
    eager = []
    for b in (b1, b2):
        y = dp.fresh_y()
        sgmv.lora_add(y, dp.x, b, p.scale, sgmv.make_workspace(n, h_in, r, dp.x.device))
        eager.append(y)
    torch.cuda.synchronize()
    for b, y, ids in zip((b1, b2), eager, (ids1, ids2)):
        ref = oracle.lora_add(p.y, p.x, ids, p.A, p.B, p.scale, p.dtype)
        _assert_close(_y_f64(y, p.dtype), ref, f"flip r={r} eager")
    ws = sgmv.make_workspace(n, h_in, r, dp.x.device)
    y1, y2 = dp.fresh_y(), dp.fresh_y()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # creates the library's side streams before the capture
        sgmv.lora_add(y1, dp.x, b1, p.scale, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sgmv.lora_add(y1, dp.x, b1, p.scale, ws)
        sgmv.lora_add(y2, dp.x, b2, p.scale, ws)
    for rep in range(4):
        y1.copy_(dp.y0)
        y2.copy_(dp.y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[graph flip] r={r} replay {rep}")
        assert torch.equal(y1, eager[0]), f"replay {rep}: first call differs from eager"
        assert torch.equal(y2, eager[1]), f"replay {rep}: second call differs from eager"
        _ = (dp.x.float() * 2).sum()
        torch.cuda.synchronize()
    assert sgmv.workspace_flags(ws) == 0


@pytest.mark.parametrize("wrong", ["max_below_16", "min_at_least_16"])
def test_segment_bounds_that_contradict_the_tables_are_flagged(torch_cuda, wrong):
    """min_seg_len / max_seg_len only choose which kernels run.  A caller bound that hides
    a segment kind leaves that kind's rows uncomputed, and the kernels that do run flag
    the workspace (SGMV_FLAG_SEG_BOUNDS); rows of the other kind are still right."""
    torch = torch_cuda
    from adapter_gemv_amd import _lib, sgmv
    # one 20-row segment and short ones (n = 40, S = 5), or one 50-row segment and a
    # 14-row one (n = 64, S = 2); both pass the host's pigeonhole check
    if wrong == "max_below_16":
        ids = np.concatenate([np.zeros(20, np.int32), np.repeat(np.arange(1, 5, dtype=np.int32), 5)])
    else:
        ids = np.concatenate([np.zeros(50, np.int32), np.ones(14, np.int32)])
    p = synth.random_problem((95, len(ids)), n=ids.size, h_in=1032, h_out=520, r=16,
                             n_adapters=5, dtype="bf16", ids=ids)
    dp = _upload(p)
    t = dp.batch.table
    lo, hi = (t.min_seg_len, 15) if wrong == "max_below_16" else (16, t.max_seg_len)
    ws = sgmv.make_workspace(p.n, p.h_in, 16, dp.x.device)
    y = dp.fresh_y()
    st = sgmv.sgmv_lora_add(sgmv._stream_handle(), _lib.BF16, y.data_ptr(), y.stride(0),
                            dp.x.data_ptr(), dp.x.stride(0), dp.batch.A_ptrs_addr,
                            dp.batch.B_ptrs_addr, dp.batch.seg_starts_addr, dp.batch.perm_addr,
                            p.n, t.n_segments, lo, hi, p.h_in, p.h_out, 16, p.scale,
                            ws.data_ptr(), ws.numel())
    assert st == _lib.OK
    torch.cuda.synchronize()
    assert sgmv.workspace_flags(ws) == _lib.FLAG_SEG_BOUNDS
    counts = np.bincount(ids)
    computed = (counts[ids] < 16) if wrong == "max_below_16" else (counts[ids] >= 16)
    got = _y_f64(y, p.dtype)
    ref = oracle.lora_add(p.y[computed], p.x[computed], p.ids[computed], p.A, p.B, p.scale,
                          p.dtype)
    _assert_close(got[computed], ref, f"bounds {wrong}: rows computed")
    assert np.array_equal(got[~computed], oracle.decode(p.y[~computed], p.dtype))
    # sgmv_check_workspace reports the flag and clears it on request
    f = np.zeros(1, np.int32)
    assert sgmv.sgmv_check_workspace(sgmv._stream_handle(), ws.data_ptr(), f.ctypes.data, 1) \
        == _lib.ERR_DEVICE
    assert int(f[0]) == _lib.FLAG_SEG_BOUNDS
    assert sgmv.workspace_flags(ws) == 0


@pytest.mark.parametrize("path", ["table", "host ids"])
def test_y_rows_past_4_gib(torch_cuda, path):
    """y rows 2^27 elements apart, so that the last of 17 rows starts 4 GiB past y's first
    byte, beyond 32-bit buffer offsets: the MFMA expand of the 16-row segment then writes y
    with plain global stores, and the decode kernel's per-row buffers each start at their
    row.  Every row against the oracle; the padding after row 0 keeps its sentinel."""
    torch = torch_cuda
    n, h_in, h_out, r = 17, 256, 264, 16
    _say(f"[y past 4 GiB] {path} n={n} h_out={h_out} ld_y=2^27")
    ids = np.array([0] * 16 + [1], dtype=np.int32)  # a 16-row segment and a 1-row segment
    p = synth.random_problem((96,), n=n, h_in=h_in, h_out=h_out, r=r, n_adapters=2, dtype="f16",
                             ids=ids)
    dp = _upload(p)
    wide = torch.empty((n, 1 << 27), dtype=torch.float16, device=dp.x.device)  # 4.25 GiB
    y = wide[:, :h_out]
    y.copy_(dp.y0)
    wide[:, h_out:h_out + 64] = -7.0
    if path == "table":
        dp.lora_add(y=y)
    else:
        dp.lora_add_host_ids(y=y)
    torch.cuda.synchronize()
    pad = wide[:, h_out:h_out + 64].cpu().numpy()
    got = _y_f64(y, "f16")
    del wide, y
    torch.cuda.empty_cache()
    assert np.all(pad == np.float16(-7.0)), f"{int((pad != np.float16(-7.0)).sum())} padding values changed"
    _assert_close(got, oracle.lora_add_problem(p), f"y past 4 GiB, {path}")
