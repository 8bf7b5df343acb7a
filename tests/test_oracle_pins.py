"""Pins of the fp64 oracle against facts that do not come from its own code.

* a hand-worked example (tests/golden/hand_example.json);
* exact rational brute force on tiny inputs (fractions.Fraction, per-element loops);
* a closed form (rank 1, A = e_k);
* invariants: B = 0 / scale = 0, linearity, splitting an adapter, row order;
* exactness of power-of-two-grid inputs;
* the I/O formats' definitions (tests/golden/io_rounding.json);
* the stable sort against numpy's stable argsort and its defining order;
* planted mistakes: mutated copies of the oracle must fail at least one pin.
"""
import json
import os
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import sgmv_oracle
from workloads import synth

DTYPES = ("f16", "bf16")


# --------------------------------------------------------------------------------------
# helpers that restate nothing of the oracle: exact rational arithmetic, element loops
# --------------------------------------------------------------------------------------
def _exact_value_f16(h):
    """Exact rational value of one binary16 number from its bit fields."""
    bits = int(np.asarray(h, np.float16).view(np.uint16))
    sign = -1 if bits >> 15 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    assert e != 0x1F
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * (Fraction(1024 + f, 1024) * (Fraction(2) ** (e - 15)))


def _exact_value_bf16(b):
    bits = int(b)
    sign = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f, 1 << 7) * (Fraction(2) ** -126)
    return sign * Fraction(128 + f, 128) * (Fraction(2) ** (e - 127))


def _exact(arr, dtype):
    fn = _exact_value_f16 if dtype == "f16" else _exact_value_bf16
    flat = [fn(v) for v in np.asarray(arr).reshape(-1)]
    return np.array(flat, dtype=object).reshape(np.asarray(arr).shape)


def brute_force(p):
    """Per-element definition in exact rationals: for each token t, with a = ids[t],
    v_j = sum_k x[t,k] A[k,j];  y'[t,c] = y[t,c] + scale * sum_j v_j B[j,c],
    where A[k, j] is stored at A_pool[a, j, k] and B[j, c] at B_pool[a, c, j]."""
    X, Y = _exact(p.x, p.dtype), _exact(p.y, p.dtype)
    Ap, Bp = _exact(p.A, p.dtype), _exact(p.B, p.dtype)
    s = Fraction(p.scale)
    out = np.empty((p.n, p.h_out), dtype=object)
    vs = np.empty((p.n, p.r), dtype=object)
    for t in range(p.n):
        a = int(p.ids[t])
        v = []
        for j in range(p.r):
            acc = Fraction(0)
            for k in range(p.h_in):
                acc += X[t, k] * Ap[a, j, k]
            v.append(acc)
        vs[t] = v
        for c in range(p.h_out):
            acc = Fraction(0)
            for j in range(p.r):
                acc += v[j] * Bp[a, c, j]
            out[t, c] = Y[t, c] + s * acc
    return vs, out


def _as_f64(obj):
    return np.array([float(v) for v in np.asarray(obj).reshape(-1)]).reshape(np.asarray(obj).shape)


def _hand_problem(dtype, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_example.json")))
    A_math = np.array(g["A_math"], np.float32)                  # [P, h_in, r]
    B_math = np.array(g["B_math"], np.float32)                  # [P, r, h_out]
    p = synth.Problem(
        "hand", dtype, np.array(g["ids"], np.int32),
        synth.quantize(np.array(g["x"], np.float32), dtype),
        synth.quantize(np.array(g["y_in"], np.float32), dtype),
        synth.quantize(np.ascontiguousarray(A_math.transpose(0, 2, 1)), dtype),
        synth.quantize(np.ascontiguousarray(B_math.transpose(0, 2, 1)), dtype),
        float(g["scale"]))
    return p, g


# --------------------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", DTYPES)
def test_hand_example(dtype, golden_dir):
    p, g = _hand_problem(dtype, golden_dir)
    assert np.array_equal(oracle.shrink(p.x, p.ids, p.A, dtype), np.array(g["v_expected"], float))
    assert np.array_equal(oracle.lora_add_problem(p), np.array(g["y_expected"], float))
    perm, starts, seg_ad = oracle.segments(p.ids, p.n_adapters)
    assert perm.tolist() == g["perm"]
    assert starts.tolist() == g["seg_starts"]
    assert seg_ad.tolist() == g["seg_adapter"]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("seed", range(4))
def test_brute_force_exact_rationals(dtype, seed):
    rng = np.random.default_rng(100 + seed)
    n, h_in, h_out, r, P = (int(rng.integers(1, 7)), int(rng.integers(1, 6)) * 8,
                            int(rng.integers(1, 6)) * 8, int(rng.integers(1, 5)),
                            int(rng.integers(1, 4)))
    p = synth.random_problem((900, seed), n=n, h_in=h_in, h_out=h_out, r=r,
                             n_adapters=P, dtype=dtype, scale=float(rng.uniform(0.25, 3)))
    v_exact, y_exact = brute_force(p)
    v = oracle.shrink(p.x, p.ids, p.A, dtype)
    y = oracle.lora_add_problem(p)
    ve, ye = _as_f64(v_exact), _as_f64(y_exact)
    assert np.all(np.abs(v - ve) <= 1e-12 * (1 + np.abs(ve)))
    assert np.all(np.abs(y - ye) <= 1e-12 * (1 + np.abs(ye)))


@pytest.mark.parametrize("dtype", DTYPES)
def test_exact_grid_inputs_are_exact(dtype):
    """On power-of-two grids the fp64 oracle must equal the exact rational result."""
    p = synth.exact_problem((7,), n=5, h_in=40, h_out=24, r=4, n_adapters=3, dtype=dtype)
    _, y_exact = brute_force(p)
    y = oracle.lora_add_problem(p)
    assert np.array_equal(y, _as_f64(y_exact))
    # and every exact value is on the 2**-8 grid and below the bound used for fp32
    assert np.all(np.abs(y) <= 255 / 256 + 2 * 40 * 2 ** -6 * 0.25 * 4)
    assert np.all(y * 256 == np.round(y * 256))


@pytest.mark.parametrize("dtype", DTYPES)
def test_closed_form_rank1(dtype):
    """r = 1 and A = e_k: the update is scale * x[:, k] * B[:, 0] (outer product)."""
    k = 5
    p = synth.random_problem((11,), n=7, h_in=32, h_out=16, r=1, n_adapters=2, dtype=dtype,
                             scale=1.5)
    A = np.zeros_like(p.A)
    one = synth.quantize(np.ones(1, np.float32), dtype)[0]
    A[:, 0, k] = one
    p.A = A
    y = oracle.lora_add_problem(p)
    X, Y = oracle.decode(p.x, dtype), oracle.decode(p.y, dtype)
    for t in range(p.n):
        b = oracle.decode(p.B[p.ids[t], :, 0], dtype)
        assert np.allclose(y[t], Y[t] + 1.5 * X[t, k] * b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", DTYPES)
def test_zero_B_and_zero_scale_leave_y(dtype):
    p = synth.random_problem((12,), n=9, h_in=64, h_out=40, r=4, n_adapters=3, dtype=dtype)
    y0 = oracle.decode(p.y, dtype)
    assert np.array_equal(oracle.lora_add(p.y, p.x, p.ids, p.A, np.zeros_like(p.B), 2.0, dtype), y0)
    assert np.array_equal(oracle.lora_add(p.y, p.x, p.ids, p.A, p.B, 0.0, dtype), y0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_linearity(dtype):
    p = synth.random_problem((13,), n=9, h_in=64, h_out=40, r=4, n_adapters=3, dtype=dtype)
    y0 = oracle.decode(p.y, dtype)
    d1 = oracle.lora_add_problem(p) - y0
    # scale: doubling the scale doubles the update
    d2 = oracle.lora_add(p.y, p.x, p.ids, p.A, p.B, 2 * p.scale, dtype) - y0
    assert np.allclose(d2, 2 * d1, rtol=1e-12, atol=1e-12)
    # x: doubling x (exact in storage) doubles v exactly and the update
    x2 = synth.quantize(oracle.decode(p.x, dtype) * 2, dtype)
    v1 = oracle.shrink(p.x, p.ids, p.A, dtype)
    v2 = oracle.shrink(x2, p.ids, p.A, dtype)
    assert np.array_equal(v2, 2 * v1)
    d3 = oracle.lora_add(p.y, x2, p.ids, p.A, p.B, p.scale, dtype) - y0
    assert np.allclose(d3, 2 * d1, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", DTYPES)
def test_identical_adapter_equals_any_split(dtype):
    """One adapter for all rows equals the same rows split over copies of it."""
    p = synth.random_problem((14,), n=12, h_in=48, h_out=32, r=4, n_adapters=1, dtype=dtype,
                             ids=np.zeros(12, np.int32))
    ref = oracle.lora_add_problem(p)
    rng = np.random.default_rng(0)
    ids = rng.integers(0, 4, size=12).astype(np.int32)
    A4, B4 = np.repeat(p.A, 4, axis=0), np.repeat(p.B, 4, axis=0)
    got = oracle.lora_add(p.y, p.x, ids, A4, B4, p.scale, dtype)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dtype", DTYPES)
def test_row_order_and_segment_order_independence(dtype):
    p = synth.random_problem((15,), n=11, h_in=48, h_out=32, r=4, n_adapters=4, dtype=dtype)
    ref = oracle.lora_add_problem(p)
    q = np.random.default_rng(1).permutation(p.n)
    got = oracle.lora_add(p.y[q], p.x[q], p.ids[q], p.A, p.B, p.scale, dtype)
    assert np.allclose(got, ref[q], rtol=1e-13, atol=1e-13)
    # relabel adapters (changes the segment order): same result
    relabel = np.array([2, 0, 3, 1], np.int32)
    A2, B2 = np.empty_like(p.A), np.empty_like(p.B)
    A2[relabel], B2[relabel] = p.A, p.B
    got2 = oracle.lora_add(p.y, p.x, relabel[p.ids], A2, B2, p.scale, dtype)
    assert np.allclose(got2, ref, rtol=1e-13, atol=1e-13)


def test_io_format_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "io_rounding.json")))
    for hexbits, val in g["bf16_decode"]:
        bits = np.array([int(hexbits, 16)], np.uint16)
        assert oracle.decode(bits, "bf16")[0] == val
    for val, hexbits in g["bf16_round"]:
        assert int(oracle.round_io(np.array([val]), "bf16")[0]) == int(hexbits, 16), val
    for val, hexbits in g["f16_round"]:
        assert int(oracle.round_io(np.array([val]), "f16").view(np.uint16)[0]) == int(hexbits, 16)


def test_round_io_bf16_matches_exact_definition():
    """Random doubles: the bf16 rounding is the nearest 8-significant-bit value (ties even)."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal(2000) * np.exp2(rng.integers(-30, 30, 2000))
    got = oracle.decode(oracle.round_io(v, "bf16"), "bf16")
    for a, b in zip(v, got):
        fa = Fraction(float(a))
        e = int(np.floor(np.log2(abs(a))))
        ulp = Fraction(2) ** (e - 7)
        lo = (fa / ulp).__floor__() * ulp
        hi = lo + ulp
        if fa - lo < hi - fa:
            want = lo
        elif fa - lo > hi - fa:
            want = hi
        else:
            want = lo if (lo / ulp) % 2 == 0 else hi
        assert Fraction(float(b)) == want


@pytest.mark.parametrize("case", ["random", "same", "distinct", "empty_adapters", "n0", "n1"])
def test_segments_definition(case):
    rng = np.random.default_rng(3)
    P = 9
    ids = {
        "random": rng.integers(0, P, 200),
        "same": np.full(50, 4),
        "distinct": rng.permutation(P),
        "empty_adapters": rng.choice([1, 5, 8], 40),
        "n0": np.zeros(0),
        "n1": np.array([7]),
    }[case].astype(np.int32)
    perm, starts, seg_ad = oracle.segments(ids, P)
    n = ids.size
    # numpy's stable argsort is the same permutation
    assert np.array_equal(perm, np.argsort(ids, kind="stable").astype(np.int32))
    # defining order: (id, caller index) strictly increasing along the sorted rows
    keys = [(int(ids[i]), int(i)) for i in perm]
    assert keys == sorted(keys) and sorted(perm.tolist()) == list(range(n))
    # segments: contiguous runs of one id, ascending ids, no empty segment
    assert starts[0] == 0 and starts[-1] == n and len(starts) == len(seg_ad) + 1
    assert np.all(np.diff(starts) > 0)
    assert np.array_equal(seg_ad, np.unique(ids).astype(np.int32))
    for s, a in enumerate(seg_ad):
        assert np.all(ids[perm[starts[s]:starts[s + 1]]] == a)


def test_segments_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.segments(np.array([0, 3], np.int32), 3)
    with pytest.raises(ValueError):
        oracle.segments(np.array([-1], np.int32), 3)


def test_ptr_table():
    base = np.array([1000, 2000, 3000, 4000], np.uint64)
    assert oracle.ptr_table(base, np.array([1, 3], np.int32)).tolist() == [2000, 4000]


# --------------------------------------------------------------------------------------
# mixed ranks
# --------------------------------------------------------------------------------------
def _ranked_tiny(dtype, seed=0):
    """Three pools of ranks 1, 2 and 3 (any r is valid for the oracle), ids over all of
    them, a different scale per rank."""
    rng = np.random.default_rng(700 + seed)
    n, h_in, h_out = 7, 16, 8
    pools = []
    for k, (P, r) in enumerate([(2, 1), (3, 2), (1, 3)]):
        q = synth.random_problem((701, seed, k), n=1, h_in=h_in, h_out=h_out, r=r,
                                 n_adapters=P, dtype=dtype)
        pools.append((q.A, q.B))
    base = synth.random_problem((702, seed), n=n, h_in=h_in, h_out=h_out, r=1, n_adapters=6,
                                dtype=dtype)
    ids = rng.integers(0, 6, n).astype(np.int32)
    scales = {1: 0.75, 2: 2.0, 3: -1.5}
    return base.x, base.y, ids, pools, scales


def brute_force_ranked(x, y, ids, pools, scales, dtype):
    """Exact rationals, row by row: the row's pool k and local index give its A, B and r,
    and the rank's scale multiplies the product."""
    out = np.empty((ids.size, y.shape[1]), dtype=object)
    off = 0
    for A_k, B_k in pools:
        P, r = A_k.shape[0], A_k.shape[1]
        for t in range(ids.size):
            if off <= ids[t] < off + P:
                row = synth.Problem("row", dtype, np.array([ids[t] - off], np.int32),
                                    x[t:t + 1], y[t:t + 1], A_k, B_k, scales[r])
                out[t] = brute_force(row)[1][0]
        off += P
    return out


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("seed", range(2))
def test_ranked_brute_force_exact_rationals(dtype, seed):
    x, y, ids, pools, scales = _ranked_tiny(dtype, seed)
    want = _as_f64(brute_force_ranked(x, y, ids, pools, scales, dtype))
    got = oracle.lora_add_ranked(y, x, ids, pools, scales, dtype)
    assert np.all(np.abs(got - want) <= 1e-12 * (1 + np.abs(want)))


@pytest.mark.parametrize("dtype", DTYPES)
def test_ranked_equals_zero_padded_single_rank(dtype):
    """Adapters of rank 16 padded with zero columns of A and zero rows of B to rank 64 give
    the same update, so with one scale for both ranks the mixed batch equals a rank-64
    batch over the padded pool."""
    p16 = synth.random_problem((703, 1), n=40, h_in=64, h_out=48, r=16, n_adapters=3,
                               dtype=dtype)
    p64 = synth.random_problem((703, 2), n=40, h_in=64, h_out=48, r=64, n_adapters=2,
                               dtype=dtype)
    ids = np.random.default_rng(704).integers(0, 5, 40).astype(np.int32)
    A16 = np.zeros((3, 64, 64), p16.A.dtype)
    A16[:, :16, :] = p16.A
    B16 = np.zeros((3, 48, 64), p16.B.dtype)
    B16[:, :, :16] = p16.B
    A = np.concatenate([A16, p64.A])
    B = np.concatenate([B16, p64.B])
    got = oracle.lora_add_ranked(p16.y, p16.x, ids, [(p16.A, p16.B), (p64.A, p64.B)],
                                 {16: 1.25, 64: 1.25}, dtype)
    want = oracle.lora_add(p16.y, p16.x, ids, A, B, 1.25, dtype)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", ["random", "one_rank", "n1", "n0"])
def test_segments_ranked_definition(case):
    rng = np.random.default_rng(9)
    rank = np.array([64, 16, 32, 16, 64, 16, 32], np.int32)
    ids = {"random": rng.integers(0, 7, 120), "one_rank": rng.choice([1, 3, 5], 30),
           "n1": np.array([4]), "n0": np.zeros(0)}[case].astype(np.int32)
    perm, groups = oracle.segments_ranked(ids, rank)
    n = ids.size
    assert sorted(perm.tolist()) == list(range(n))
    keys = [(int(rank[ids[i]]), int(ids[i]), int(i)) for i in perm]
    assert all(keys[i] < keys[i + 1] for i in range(n - 1))
    assert [g[0] for g in groups] == sorted(set(int(rank[a]) for a in ids))
    row = 0
    for r, row0, gn, starts, seg_ad in groups:
        assert row0 == row and starts[0] == 0 and starts[-1] == gn and np.all(np.diff(starts) > 0)
        for s, a in enumerate(seg_ad):
            rows = perm[row0 + starts[s]: row0 + starts[s + 1]]
            assert rank[a] == r and np.all(ids[rows] == a)
        assert np.array_equal(seg_ad, np.unique(ids[perm[row0:row0 + gn]]))
        row += gn
    assert row == n


# --------------------------------------------------------------------------------------
# planted mistakes: a mutated oracle must fail at least one pin
# --------------------------------------------------------------------------------------
MUTATIONS = [
    ("drop scale", "float(scale) * (", "1.0 * ("),
    ("wrong adapter for A", "A64[int(a)]", "A64[(int(a) + 1) % A64.shape[0]]"),
    ("B not transposed", "@ B_a.T)", "@ B_a)"),
    ("sign", "out[rows] += float(scale)", "out[rows] -= float(scale)"),
    ("unstable sort", "for i, t in enumerate(ids):", "for i, t in reversed(list(enumerate(ids))):"),
    ("bf16 shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("round toward zero", "np.rint(np.ldexp(m, 8))", "np.trunc(np.ldexp(m, 8))"),
    ("y not added", "out = Y.copy()", "out = np.zeros_like(Y)"),
    ("ranked: one scale for every rank", "B_k, scales[r], dtype)", "B_k, scales[min(scales)], dtype)"),
    ("ranked: pools not offset", "        off += P\n    return out", "        off += 0\n    return out"),
    ("ranked: rank not the leading key", "keys = [(int(rank[a]), int(a), t)", "keys = [(0 * int(rank[a]), int(a), t)"),
]


def _mutant(old, new):
    src = open(sgmv_oracle.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("mutant_oracle")
    exec(compile(src.replace(old, new), "mutant_oracle", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod, golden_dir):
    try:
        for dtype in DTYPES:
            p, g = _hand_problem(dtype, golden_dir)
            if not np.array_equal(mod.lora_add(p.y, p.x, p.ids, p.A, p.B, p.scale, dtype),
                                  np.array(g["y_expected"], float)):
                return False
            perm, _, _ = mod.segments(p.ids, p.n_adapters)
            if perm.tolist() != g["perm"]:
                return False
        gi = json.load(open(os.path.join(golden_dir, "io_rounding.json")))
        for hexbits, val in gi["bf16_decode"]:
            if mod.decode(np.array([int(hexbits, 16)], np.uint16), "bf16")[0] != val:
                return False
        for val, hexbits in gi["bf16_round"]:
            if int(mod.round_io(np.array([val]), "bf16")[0]) != int(hexbits, 16):
                return False
        ids = np.array([2, 0, 2, 1, 0, 2], np.int32)
        perm, _, _ = mod.segments(ids, 3)
        if not np.array_equal(perm, np.argsort(ids, kind="stable")):
            return False
        x, y, rids, pools, scales = _ranked_tiny("bf16")
        want = _as_f64(brute_force_ranked(x, y, rids, pools, scales, "bf16"))
        if not np.allclose(mod.lora_add_ranked(y, x, rids, pools, scales, "bf16"), want,
                           rtol=1e-12, atol=1e-12):
            return False
        perm, groups = mod.segments_ranked(np.array([0, 1, 0, 2], np.int32),
                                           np.array([64, 16, 32], np.int32))
        if perm.tolist() != [1, 3, 0, 2] or [g[0] for g in groups] != [16, 32, 64]:
            return False
    except Exception:
        return False
    return True


def test_pins_pass_on_the_real_oracle(golden_dir):
    assert _pins_pass(sgmv_oracle, golden_dir)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, golden_dir):
    assert not _pins_pass(_mutant(old, new), golden_dir), name
