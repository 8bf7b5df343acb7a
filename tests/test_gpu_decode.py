"""GPU tests of the one-launch decode path (sgmv_lora_add_pool, sgmv_build_segments_device):
device segment metadata bit-exact against the oracle's stable sort, parity of y against
the fp64 oracle, bit-exact grids and gather probes, invalid ids, counter self-reset and
HIP graph replay."""
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


def _upload(p):
    from adapter_gemv_amd.device_problem import DeviceProblem
    return DeviceProblem.upload(p)


def _storage(y, dtype):
    from adapter_gemv_amd.device_problem import to_numpy_storage
    return to_numpy_storage(y, dtype)


def _assert_close(got, ref, what):
    err = np.abs(got - ref)
    tol = 1e-2 + 1e-2 * np.abs(ref)
    _say(f"{what}: max|err| {err.max():.3e}, worst err/tol {np.max(err / tol):.3f}")
    assert np.all(err <= tol), f"{what}: {int((err > tol).sum())} outside tolerance"


ID_CASES = [
    ("n1", np.array([3], np.int32), 5),
    ("distinct32", np.random.default_rng(0).permutation(32).astype(np.int32), 32),
    ("same64", np.full(64, 7, np.int32), 9),
    ("uniform64", np.random.default_rng(1).integers(0, 64, 64).astype(np.int32), 64),
    ("zipf40", synth.truncated_zipf_ids(np.random.default_rng(2), 40, 4096, 1.2), 4096),
    ("sparse_pool", np.random.default_rng(3).choice([5, 900, 4000], 33).astype(np.int32), 4096),
    # the one-workgroup device sort (n > 64)
    ("n65", np.random.default_rng(4).integers(0, 9, 65).astype(np.int32), 9),
    ("uniform300", np.random.default_rng(5).integers(0, 300, 300).astype(np.int32), 300),
    ("zipf1000", synth.truncated_zipf_ids(np.random.default_rng(6), 1000, 5000, 1.1), 5000),
    ("distinct4096", np.random.default_rng(7).permutation(4096).astype(np.int32), 4096),
    ("same4096", np.full(4096, 3, np.int32), 4),
    ("mixed70b", synth.mixed70b_ids(np.random.default_rng(8)), 50),
    ("big_ids", np.random.default_rng(9).choice([0, 1 << 19, (1 << 20) - 1], 777).astype(np.int32),
     1 << 20),
]


@pytest.mark.parametrize("name,ids,P", ID_CASES, ids=[c[0] for c in ID_CASES])
def test_device_segments_match_oracle(torch_cuda, name, ids, P):
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    _say(f"[segments] {name}")
    d = torch.as_tensor(ids, device="cuda")
    perm, starts, seg_ad, S = sgmv.build_segments_device(d, P)
    torch.cuda.synchronize()
    rp, rs, ra = oracle.segments(ids, P)
    s = int(S.item())
    assert s == len(ra)
    assert np.array_equal(perm.cpu().numpy()[: len(ids)], rp)
    assert np.array_equal(starts.cpu().numpy()[: s + 1], rs)
    assert np.array_equal(seg_ad.cpu().numpy()[:s], ra)


def test_device_segments_flag_bad_ids(torch_cuda):
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    d = torch.as_tensor(np.array([0, 5, 1], np.int32), device="cuda")
    _, _, _, S = sgmv.build_segments_device(d, 3)
    assert int(S.item()) == -1
    # large sort: the valid rows are still sorted and the rest of perm is -1
    ids = np.random.default_rng(10).integers(0, 6, 500).astype(np.int32)
    ids[[7, 123, 499]] = [6, -2, 100]
    perm, starts, seg_ad, S = sgmv.build_segments_device(torch.as_tensor(ids, device="cuda"), 6)
    torch.cuda.synchronize()
    assert int(S.item()) == -1
    keep = (ids >= 0) & (ids < 6)
    rp, rs, ra = oracle.segments(np.where(keep, ids, 0).astype(np.int32)[keep], 6)
    rows = np.flatnonzero(keep)
    got = perm.cpu().numpy()
    assert np.array_equal(got[: keep.sum()], rows[rp])
    assert np.all(got[keep.sum():] == -1)
    assert np.array_equal(starts.cpu().numpy()[: len(ra) + 1], rs)
    assert np.array_equal(seg_ad.cpu().numpy()[: len(ra)], ra)


DECODE = ["tiny", "decode7b", "sweep_a", "sweep_b", "sweep_c"]
FACT = dict(synth.all_workloads())


@pytest.mark.parametrize("name", DECODE)
def test_decode_workloads(torch_cuda, name):
    _say(f"[pool parity] {name}")
    p = FACT[name]()
    dp = _upload(p)
    y = dp.lora_add_pool()
    torch_cuda.cuda.synchronize()
    _assert_close(oracle.decode(_storage(y, p.dtype), p.dtype), oracle.lora_add_problem(p), name)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("r", [16, 32, 64])
@pytest.mark.parametrize("n,P,kind", [(1, 3, "u"), (32, 32, "perm"), (64, 5, "u"), (47, 40, "zipf")])
def test_pool_exact_bit_exact(torch_cuda, dtype, r, n, P, kind):
    _say(f"[pool exact] n={n} P={P} r={r} {dtype}")
    rng = np.random.default_rng(n * 100 + r)
    ids = {"u": rng.integers(0, P, n), "perm": rng.permutation(n) % P,
           "zipf": synth.truncated_zipf_ids(rng, n, P, 1.2)}[kind].astype(np.int32)
    p = synth.exact_problem((81, n, r), n=n, h_in=2056, h_out=1544, r=r, n_adapters=P,
                            dtype=dtype, ids=ids)
    y = _upload(p).lora_add_pool()
    torch_cuda.cuda.synchronize()
    got = _storage(y, dtype).view(np.uint16)
    want = oracle.round_io(oracle.lora_add_problem(p), dtype).view(np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("r", [16, 64])
def test_pool_gather_probe(torch_cuda, dtype, r):
    _say(f"[pool gather] r={r} {dtype}")
    rng = np.random.default_rng(r)
    ids = rng.integers(0, 6, 50).astype(np.int32)
    p = synth.gather_probe((82, r), n=50, h_in=512, h_out=384, r=r, n_adapters=6, dtype=dtype,
                           ids=ids)
    y = _upload(p).lora_add_pool()
    torch_cuda.cuda.synchronize()
    want = oracle.round_io(oracle.lora_add_problem(p), dtype).view(np.uint16)
    assert np.array_equal(_storage(y, dtype).view(np.uint16), want)


RAGGED = [(5, 8, 8, 16), (33, 200, 136, 16), (64, 4104, 1032, 32), (17, 24, 4104, 64),
          (60, 28672, 8192, 16), (12, 8192, 1024, 64)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n,h_in,h_out,r", RAGGED)
def test_pool_ragged(torch_cuda, dtype, n, h_in, h_out, r):
    _say(f"[pool ragged] n={n} {h_in}x{h_out} r={r} {dtype}")
    p = synth.random_problem((83, n, h_in, h_out), n=n, h_in=h_in, h_out=h_out, r=r,
                             n_adapters=7, dtype=dtype, id_dist="zipf", zipf_s=1.1, scale=1.25)
    y = _upload(p).lora_add_pool()
    torch_cuda.cuda.synchronize()
    _assert_close(oracle.decode(_storage(y, dtype), dtype), oracle.lora_add_problem(p),
                  f"ragged n={n} {h_in}x{h_out} r={r}")


def test_pool_invalid_ids_skip_rows_and_flag(torch_cuda):
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    p = synth.random_problem((84,), n=20, h_in=256, h_out=128, r=16, n_adapters=4, dtype="f16")
    dp = _upload(p)
    ids = p.ids.copy()
    ids[[3, 11]] = [4, -1]
    ws = sgmv.make_workspace(p.n, p.h_in, 16, dp.x.device)
    y = dp.lora_add_pool(ids=torch.as_tensor(ids, device="cuda"), workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 2
    got = oracle.decode(_storage(y, "f16"), "f16")
    keep = np.ones(p.n, bool)
    keep[[3, 11]] = False
    ref = oracle.lora_add(p.y[keep], p.x[keep], p.ids[keep], p.A, p.B, p.scale, "f16")
    _assert_close(got[keep], ref, "valid rows")
    assert np.array_equal(got[~keep], oracle.decode(p.y[~keep], "f16"))


def test_pool_repeat_calls_reset_counters(torch_cuda):
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    p = FACT["decode7b"]()
    dp = _upload(p)
    ws = sgmv.make_workspace(p.n, p.h_in, 16, dp.x.device)
    outs = [dp.lora_add_pool(workspace=ws) for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    assert int(ws[:16640].view(torch.int32).abs().sum().item()) == 0  # flag and counters at zero
    # the tagged partial sums (the end of the workspace, laid out for 64 rows) are left
    # at zero too
    ks = -(-p.h_in // (8192 // 16))
    tail = 8 * ks * 64 * 16 + 256
    assert int(ws[-tail:].view(torch.int32).abs().sum().item()) == 0
    # the table path on the same workspace agrees within tolerance, and a decode-path call
    # after it still gives the same bits
    y2 = dp.lora_add(workspace=ws)
    torch.cuda.synchronize()
    _assert_close(oracle.decode(_storage(y2, "f16"), "f16"),
                  oracle.decode(_storage(outs[0], "f16"), "f16"), "pool vs table path")
    y3 = dp.lora_add_pool(workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y3, outs[0])


def test_pool_hip_graph_replay(torch_cuda):
    """Capture several calls (different ids and y buffers) in one HIP graph and replay it
    a few times, with eager work between replays; every replay must match eager."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    p = FACT["decode7b"]()
    dp = _upload(p)
    ws = sgmv.make_workspace(p.n, p.h_in, 16, dp.x.device)
    rng = np.random.default_rng(5)
    id_sets = [torch.as_tensor(rng.permutation(32).astype(np.int32), device="cuda") for _ in range(3)]
    ys = [dp.fresh_y() for _ in range(3)]
    # eager reference of one pass over the three calls
    ref = [dp.fresh_y() for _ in range(3)]
    for k in range(3):
        sgmv.lora_add_pool(ref[k], dp.x, id_sets[k], dp.A, dp.B, p.scale, ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm the capture stream
        for k in range(3):
            sgmv.lora_add_pool(dp.fresh_y(), dp.x, id_sets[k], dp.A, dp.B, p.scale, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(3):
            sgmv.lora_add_pool(ys[k], dp.x, id_sets[k], dp.A, dp.B, p.scale, ws)
    for rep in range(3):
        for k in range(3):
            ys[k].copy_(dp.y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(3):
            assert torch.equal(ys[k], ref[k]), f"replay {rep} call {k}"
        _ = (dp.x.float() * 2).sum()                 # eager work between replays
        torch.cuda.synchronize()
    assert int(ws[:16640].view(torch.int32).abs().sum().item()) == 0


def test_shared_workspace_across_shapes(torch_cuda):
    """One workspace sized for the largest call serves decode-path calls of varying n and
    h_in interleaved with table-path calls whose scratch is larger: every result matches
    the oracle, and each decode call gives the same bits as on a fresh workspace."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    big = synth.random_problem((85, 1), n=600, h_in=5120, h_out=1032, r=16, n_adapters=3,
                               dtype="bf16", id_dist="uniform")
    dec = [synth.random_problem((85, 2, n, h), n=n, h_in=h, h_out=1032, r=16, n_adapters=40,
                                dtype="bf16", id_dist="zipf", zipf_s=1.1)
           for n, h in [(32, 4096), (17, 2048), (64, 5120), (5, 4096)]]
    ws = sgmv.make_workspace(big.n, big.h_in, 16, torch.device("cuda"))
    for rep in range(2):
        for q in dec:
            _say(f"[shared ws] rep {rep} decode n={q.n} h_in={q.h_in}")
            dq = _upload(q)
            y = dq.lora_add_pool(workspace=ws)
            torch.cuda.synchronize()
            fresh = dq.lora_add_pool()
            torch.cuda.synchronize()
            assert torch.equal(y, fresh)
            _assert_close(oracle.decode(_storage(y, "bf16"), "bf16"), oracle.lora_add_problem(q),
                          f"shared ws decode n={q.n}")
            _say(f"[shared ws] rep {rep} table n={big.n}")
            db = _upload(big)
            yb = db.lora_add(workspace=ws)
            torch.cuda.synchronize()
            _assert_close(oracle.decode(_storage(yb, "bf16"), "bf16"), oracle.lora_add_problem(big),
                          "shared ws table")
    assert int(ws[:16640].view(torch.int32).abs().sum().item()) == 0


def test_shared_workspace_table_shapes(torch_cuda):
    """Table-path calls of different n, h_in and r (host tables and device-sorted tables)
    share one workspace sized for the largest: each gives the same bits as on a fresh
    workspace, the results match the oracle, and the counters and tagged partials are
    zero afterwards."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    big = synth.random_problem((86, 1), n=2048, h_in=5120, h_out=1032, r=64, n_adapters=4,
                               dtype="bf16", ids=np.repeat(np.int32([2, 0, 3, 1]), 512))
    probs = [
        synth.random_problem((86, 2), n=64, h_in=4096, h_out=776, r=16, n_adapters=40,
                             dtype="bf16", id_dist="zipf", zipf_s=1.1),
        big,
        synth.random_problem((86, 3), n=300, h_in=2048, h_out=1032, r=32, n_adapters=7,
                             dtype="bf16", id_dist="uniform"),
    ]
    dev = [_upload(q) for q in probs]
    fresh = []
    for q, d in zip(probs, dev):
        fresh.append((d.lora_add(), d.lora_add_pool()))
        torch.cuda.synchronize()
        _assert_close(oracle.decode(_storage(fresh[-1][0], "bf16"), "bf16"),
                      oracle.lora_add_problem(q), f"fresh ws n={q.n}")
    ws = sgmv.make_workspace(big.n, big.h_in, 64, torch.device("cuda"))
    for rep in range(2):
        for q, d, (f_tab, f_pool) in zip(probs, dev, fresh):
            _say(f"[shared ws tables] rep {rep} n={q.n} h_in={q.h_in} r={q.r}")
            y = d.lora_add(workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(y, f_tab)
            y = d.lora_add_pool(workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(y, f_pool)
    assert int(ws[:16640].view(torch.int32).abs().sum().item()) == 0
    # the largest call's tagged partials: the last 8 * ceil(h_in / (8192 / r)) * 64 * r bytes
    tail = 8 * (-(-big.h_in // (8192 // 64))) * 64 * 64
    assert int(ws[-tail:].view(torch.int32).abs().sum().item()) == 0


# --------------------------------------------------------------------------------------
# device ids, 64 < n <= 4096: device sort + table kernels
# --------------------------------------------------------------------------------------
LARGE = [
    # name, n, h_in, h_out, r, P, ids kind, dtype
    ("prefill_blocks", 512, 1032, 776, 16, 4, "blocks", "bf16"),
    ("mixed_r64", 520, 1024, 1160, 64, 50, "mixed70b", "bf16"),
    ("many_short", 1000, 520, 264, 32, 500, "uniform", "f16"),
    ("one_long", 4096, 264, 136, 16, 1, "blocks", "f16"),
    ("ragged_r16", 333, 200, 3000, 16, 7, "zipf", "bf16"),
]


def _large_ids(kind, n, P, rng):
    if kind == "blocks":
        return np.repeat(rng.permutation(P), -(-n // P))[:n].astype(np.int32)
    if kind == "uniform":
        return rng.integers(0, P, n).astype(np.int32)
    if kind == "zipf":
        return synth.truncated_zipf_ids(rng, n, P, 1.1)
    dec = synth.truncated_zipf_ids(rng, 64, P - 2, 1.2)
    half = (n - 64) // 2
    return np.concatenate([dec, np.full(half, P - 2, np.int32),
                           np.full(n - 64 - half, P - 1, np.int32)]).astype(np.int32)


@pytest.mark.parametrize("case", LARGE, ids=[c[0] for c in LARGE])
def test_pool_large_batches(torch_cuda, case):
    name, n, h_in, h_out, r, P, kind, dtype = case
    _say(f"[pool large] {case}")
    ids = _large_ids(kind, n, P, np.random.default_rng(n + r))
    p = synth.random_problem((86, n, r), n=n, h_in=h_in, h_out=h_out, r=r, n_adapters=P,
                             dtype=dtype, ids=ids, scale=1.5)
    y = _upload(p).lora_add_pool()
    torch_cuda.cuda.synchronize()
    _assert_close(oracle.decode(_storage(y, dtype), dtype), oracle.lora_add_problem(p),
                  f"pool large {name}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("r,kind,n", [(16, "mixed70b", 300), (32, "blocks", 256),
                                      (64, "uniform", 200)])
def test_pool_large_exact_bit_exact(torch_cuda, dtype, r, kind, n):
    _say(f"[pool large exact] r={r} {kind} n={n} {dtype}")
    P = 12
    ids = _large_ids(kind, n, P, np.random.default_rng(3 * n + r))
    p = synth.exact_problem((87, n, r), n=n, h_in=1032, h_out=648, r=r, n_adapters=P,
                            dtype=dtype, ids=ids)
    y = _upload(p).lora_add_pool()
    torch_cuda.cuda.synchronize()
    want = oracle.round_io(oracle.lora_add_problem(p), dtype).view(np.uint16)
    assert np.array_equal(_storage(y, dtype).view(np.uint16), want)


@pytest.mark.parametrize("name", [f"prefill13b_{p}" for p in synth.PREFILL13B_SHAPES])
def test_pool_large_full_workloads(torch_cuda, name):
    """The full prefill batches with device ids (2048 rows), every row against the oracle
    (the 70B mixed batch with device ids is compared in full with its host-table run)."""
    from parity_util import compare_all_rows
    _say(f"[pool large full] {name}")
    p = FACT[name]()
    y = _upload(p).lora_add_pool()
    torch_cuda.cuda.synchronize()
    compare_all_rows({"device ids": _storage(y, p.dtype)}, p.n,
                     lambda rows: oracle.lora_add(p.y[rows], p.x[rows], p.ids[rows], p.A, p.B,
                                                  p.scale, p.dtype), p.dtype, name)


def test_pool_large_invalid_ids(torch_cuda):
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    p = synth.random_problem((88,), n=400, h_in=520, h_out=264, r=16, n_adapters=5,
                             dtype="bf16", id_dist="uniform")
    dp = _upload(p)
    ids = p.ids.copy()
    bad = [0, 17, 399]
    ids[bad] = [5, -1, 70000]
    ws = sgmv.make_workspace(p.n, p.h_in, 16, dp.x.device)
    y = dp.lora_add_pool(ids=torch.as_tensor(ids, device="cuda"), workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 2
    keep = np.ones(p.n, bool)
    keep[bad] = False
    got = oracle.decode(_storage(y, "bf16"), "bf16")
    ref = oracle.lora_add(p.y[keep], p.x[keep], p.ids[keep], p.A, p.B, p.scale, "bf16")
    _assert_close(got[keep], ref, "large valid rows")
    assert np.array_equal(got[~keep], oracle.decode(p.y[~keep], "bf16"))


def test_pool_large_hip_graph_replay(torch_cuda):
    """Capture large device-id calls (device sort + table kernels) in one HIP graph;
    every replay, with eager work between replays, must match the eager result."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    p = synth.random_problem((89,), n=700, h_in=1032, h_out=776, r=16, n_adapters=9,
                             dtype="bf16", id_dist="zipf", zipf_s=1.3)
    dp = _upload(p)
    ws = sgmv.make_workspace(p.n, p.h_in, 16, dp.x.device)
    rng = np.random.default_rng(12)
    id_sets = [torch.as_tensor(synth.truncated_zipf_ids(rng, p.n, 9, s), device="cuda")
               for s in (0.8, 1.3, 2.0)]
    ys = [dp.fresh_y() for _ in range(3)]
    ref = [dp.fresh_y() for _ in range(3)]
    for k in range(3):
        sgmv.lora_add_pool(ref[k], dp.x, id_sets[k], dp.A, dp.B, p.scale, ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(3):
            sgmv.lora_add_pool(dp.fresh_y(), dp.x, id_sets[k], dp.A, dp.B, p.scale, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(3):
            sgmv.lora_add_pool(ys[k], dp.x, id_sets[k], dp.A, dp.B, p.scale, ws)
    for rep in range(3):
        for k in range(3):
            ys[k].copy_(dp.y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(3):
            assert torch.equal(ys[k], ref[k]), f"replay {rep} call {k}"
        _ = (dp.x.float() * 2).sum()
        torch.cuda.synchronize()
    assert int(ws[:16640].view(torch.int32).abs().sum().item()) == 0


# ------------------------------------------------------------------------------------
# host ids in the kernel arguments (sgmv_lora_add_host_ids)
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", DECODE)
def test_host_ids_decode_workloads(torch_cuda, name):
    _say(f"[host-id parity] {name}")
    p = FACT[name]()
    dp = _upload(p)
    y = dp.lora_add_host_ids()
    y_dev = dp.lora_add_pool()
    torch_cuda.cuda.synchronize()
    _assert_close(oracle.decode(_storage(y, p.dtype), p.dtype), oracle.lora_add_problem(p), name)
    # the same kernel body as the device-id path: the same bits
    assert torch_cuda.equal(y, y_dev)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("r", [16, 32, 64])
@pytest.mark.parametrize("n,P,kind", [(1, 3, "u"), (64, 5, "u"), (47, 40, "zipf")])
def test_host_ids_exact_bit_exact(torch_cuda, dtype, r, n, P, kind):
    _say(f"[host-id exact] n={n} P={P} r={r} {dtype}")
    rng = np.random.default_rng(n * 100 + r + 7)
    ids = {"u": rng.integers(0, P, n), "zipf": synth.truncated_zipf_ids(rng, n, P, 1.2)}[kind]
    p = synth.exact_problem((91, n, r), n=n, h_in=2056, h_out=1544, r=r, n_adapters=P,
                            dtype=dtype, ids=ids.astype(np.int32))
    y = _upload(p).lora_add_host_ids()
    torch_cuda.cuda.synchronize()
    want = oracle.round_io(oracle.lora_add_problem(p), dtype).view(np.uint16)
    assert np.array_equal(_storage(y, dtype).view(np.uint16), want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_host_ids_gather_probe(torch_cuda, dtype):
    _say(f"[host-id gather] {dtype}")
    rng = np.random.default_rng(17)
    ids = rng.integers(0, 6, 50).astype(np.int32)
    p = synth.gather_probe((92,), n=50, h_in=512, h_out=384, r=16, n_adapters=6, dtype=dtype,
                           ids=ids)
    y = _upload(p).lora_add_host_ids()
    torch_cuda.cuda.synchronize()
    want = oracle.round_io(oracle.lora_add_problem(p), dtype).view(np.uint16)
    assert np.array_equal(_storage(y, dtype).view(np.uint16), want)


@pytest.mark.parametrize("n,h_in,h_out,r", [(33, 200, 136, 16), (17, 24, 4104, 64),
                                            (60, 28672, 8192, 16)])
def test_host_ids_ragged(torch_cuda, n, h_in, h_out, r):
    _say(f"[host-id ragged] n={n} {h_in}x{h_out} r={r}")
    p = synth.random_problem((93, n, h_in, h_out), n=n, h_in=h_in, h_out=h_out, r=r,
                             n_adapters=7, dtype="bf16", id_dist="zipf", zipf_s=1.1, scale=1.25)
    y = _upload(p).lora_add_host_ids()
    torch_cuda.cuda.synchronize()
    _assert_close(oracle.decode(_storage(y, "bf16"), "bf16"), oracle.lora_add_problem(p),
                  f"host-id ragged n={n} {h_in}x{h_out} r={r}")


@pytest.mark.parametrize("path", ["host ids", "device ids"])
def test_decode_longest_b_delay(torch_cuda, path):
    """64 tokens on 64 distinct adapters at r = 64, h_in = 4096: the shrink items fetch
    32.5 MiB, so the expand items' wait before their loads of B is at its cap; a ragged
    h_out (1032) leaves the last expand item 8 columns."""
    _say(f"[decode longest B delay] {path}")
    p = synth.random_problem((94,), n=64, h_in=4096, h_out=1032, r=64, n_adapters=64,
                             dtype="f16", ids=np.random.default_rng(94).permutation(64).astype(np.int32),
                             scale=0.5)
    dp = _upload(p)
    y = dp.lora_add_host_ids() if path == "host ids" else dp.lora_add_pool()
    torch_cuda.cuda.synchronize()
    _assert_close(oracle.decode(_storage(y, "f16"), "f16"), oracle.lora_add_problem(p),
                  f"longest B delay, {path}")


def test_host_ids_graph_replay_and_shared_workspace(torch_cuda):
    """Calls captured with different host ids replay with the ids they were captured with,
    every replay equal to eager; the workspace is shared with the device-id path and left
    at zero."""
    torch = torch_cuda
    from adapter_gemv_amd import sgmv
    p = FACT["decode7b"]()
    dp = _upload(p)
    ws = sgmv.make_workspace(p.n, p.h_in, 16, dp.x.device)
    rng = np.random.default_rng(6)
    id_sets = [rng.permutation(32).astype(np.int32) for _ in range(3)]
    ref = [dp.fresh_y() for _ in range(3)]
    for k in range(3):
        sgmv.lora_add_pool(ref[k], dp.x, torch.as_tensor(id_sets[k], device="cuda"), dp.A, dp.B,
                           p.scale, ws)
    torch.cuda.synchronize()
    ys = [dp.fresh_y() for _ in range(3)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for k in range(3):
            sgmv.lora_add_host_ids(dp.fresh_y(), dp.x, id_sets[k], dp.A, dp.B, p.scale, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(3):
            sgmv.lora_add_host_ids(ys[k], dp.x, id_sets[k], dp.A, dp.B, p.scale, ws)
    id_sets[0][:] = 0  # the captured call keeps the ids it was captured with
    for rep in range(3):
        for k in range(3):
            ys[k].copy_(dp.y0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(3):
            assert torch.equal(ys[k], ref[k]), f"replay {rep} call {k}"
        _ = (dp.x.float() * 2).sum()
        torch.cuda.synchronize()
    assert int(ws[:16640].view(torch.int32).abs().sum().item()) == 0
    ks = -(-p.h_in // (8192 // 16))
    tail = 8 * ks * 64 * 16 + 256
    assert int(ws[-tail:].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("path", ["host ids", "device ids"])
@pytest.mark.parametrize("n,h_out,r", [(40, 1032, 64), (33, 136, 16), (9, 776, 32)])
def test_decode_padded_rows_keep_their_padding(torch_cuda, path, n, h_out, r):
    """y rows wider than h_out (ld_y = h_out + 64), with an h_out that leaves the last
    expand item a partial column range: the columns past h_out hold a sentinel that the
    call must leave bit for bit, and y itself matches the oracle."""
    torch = torch_cuda
    _say(f"[decode padded rows] {path} n={n} h_out={h_out} r={r}")
    p = synth.random_problem((95, n, h_out, r), n=n, h_in=520, h_out=h_out, r=r, n_adapters=11,
                             dtype="f16", id_dist="zipf", zipf_s=1.1)
    dp = _upload(p)
    pad = 64
    wide = torch.full((n, h_out + pad), -7.0, dtype=torch.float16, device=dp.x.device)
    wide[:, :h_out] = dp.y0
    y = wide[:, :h_out]
    if path == "host ids":
        dp.lora_add_host_ids(y=y)
    else:
        dp.lora_add_pool(y=y)
    torch.cuda.synchronize()
    tail = wide[:, h_out:].cpu().numpy()
    assert np.all(tail == np.float16(-7.0)), f"{int((tail != np.float16(-7.0)).sum())} padding values changed"
    _assert_close(oracle.decode(_storage(y, "f16"), "f16"), oracle.lora_add_problem(p),
                  f"padded rows, {path}")
