"""Seeded synthetic inputs for SGMV (segmented gather matrix-vector multiplication).

This module only draws random numbers and stores them in the I/O formats; it holds
none of the method's arithmetic (no products, no sorting, no segment tables). Both
the fp64 oracle and the GPU path take their inputs from here.

Storage formats (shared by every consumer):

* ``"f16"``  arrays are ``numpy.float16``;
* ``"bf16"`` arrays are ``numpy.uint16`` holding bfloat16 bit patterns (numpy has no
  bfloat16 type); values are rounded from float32 to nearest, ties to even.

Adapter layouts.  The LoRA update of the Punica pages (project overview, "How It
Works": the pretrained W is augmented by two smaller matrices A and B) is applied as
``y += scale * (x @ A) @ B`` with A of shape ``h_in x r`` and B of shape ``r x h_out``.
Both matrices are stored so that the contracted dimension is contiguous:

* ``A_pool[a]`` has shape ``[r, h_in]``  (row j is column j of A);
* ``B_pool[a]`` has shape ``[h_out, r]`` (row c is column c of B).

This is the layout PyTorch's ``nn.Linear`` uses for the down and up projection
weights of a LoRA pair.

Distributions (per workload description): x ~ N(0, 1), y ~ N(0, 1),
A ~ N(0, std = 1/sqrt(h_in)), B ~ N(0, std = 1/sqrt(r)); adapter ids are either a
seeded permutation, uniform draws, or truncated Zipf draws over a pool.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

F16 = "f16"
BF16 = "bf16"
DTYPES = (F16, BF16)


# --------------------------------------------------------------------------------------
# storage conversions (input quantisation only)
# --------------------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def quantize(a: np.ndarray, dtype: str) -> np.ndarray:
    """Store a float array in the I/O format ``dtype`` (round to nearest even)."""
    if dtype == F16:
        return np.asarray(a, dtype=np.float32).astype(np.float16)
    if dtype == BF16:
        return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_dtype(dtype: str):
    return np.float16 if dtype == F16 else np.uint16


# --------------------------------------------------------------------------------------
# problems
# --------------------------------------------------------------------------------------
@dataclasses.dataclass
class Problem:
    """One SGMV call: ``y[t] += scale * (x[t] @ A[ids[t]]) @ B[ids[t]]`` for every row t."""

    name: str
    dtype: str
    ids: np.ndarray          # int32 [n], caller row order
    x: np.ndarray            # [n, h_in]
    y: np.ndarray            # [n, h_out] (input value; never modified here)
    A: np.ndarray            # [P, r, h_in]
    B: np.ndarray            # [P, h_out, r]
    scale: float

    @property
    def n(self) -> int:
        return int(self.ids.shape[0])

    @property
    def h_in(self) -> int:
        return int(self.x.shape[1])

    @property
    def h_out(self) -> int:
        return int(self.y.shape[1])

    @property
    def r(self) -> int:
        return int(self.A.shape[1])

    @property
    def n_adapters(self) -> int:
        return int(self.A.shape[0])

    def distinct_adapters(self) -> int:
        return int(np.unique(self.ids).size) if self.n else 0


def _streams(seed: Sequence[int], k: int = 5) -> List[np.random.Generator]:
    """Independent child generators (ids, x, y, A, B) from one seed tuple."""
    ss = np.random.SeedSequence(list(seed))
    return [np.random.default_rng(c) for c in ss.spawn(k)]


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def truncated_zipf_ids(rng: np.random.Generator, n: int, pool: int, s: float) -> np.ndarray:
    """Adapter ids drawn per token with P(id = k-1) proportional to k**-s, k = 1..pool."""
    p = np.arange(1, pool + 1, dtype=np.float64) ** (-float(s))
    p /= p.sum()
    return rng.choice(pool, size=n, p=p).astype(np.int32)


def random_problem(seed: Sequence[int], *, n: int, h_in: int, h_out: int, r: int,
                   n_adapters: int, dtype: str, scale: float = 2.0,
                   ids: Optional[np.ndarray] = None, id_dist: str = "uniform",
                   zipf_s: float = 1.5, name: str = "random") -> Problem:
    """A problem with the workload distributions and arbitrary (possibly ragged) sizes."""
    g_ids, g_x, g_y, g_a, g_b = _streams(seed)
    if ids is None:
        if id_dist == "uniform":
            ids = g_ids.integers(0, n_adapters, size=n, dtype=np.int32)
        elif id_dist == "zipf":
            ids = truncated_zipf_ids(g_ids, n, n_adapters, zipf_s)
        elif id_dist == "permutation":
            assert n == n_adapters
            ids = g_ids.permutation(n_adapters).astype(np.int32)
        else:
            raise ValueError(id_dist)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    x = quantize(_normal(g_x, (n, h_in), 1.0), dtype)
    y = quantize(_normal(g_y, (n, h_out), 1.0), dtype)
    A = quantize(_normal(g_a, (n_adapters, r, h_in), 1.0 / np.sqrt(h_in)), dtype)
    B = quantize(_normal(g_b, (n_adapters, h_out, r), 1.0 / np.sqrt(r)), dtype)
    return Problem(name, dtype, ids, x, y, A, B, float(scale))


# --------------------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------------------
def tiny() -> Problem:
    """h_in = h_out = 4096, r = 16, 4 tokens in segments [2, 2] over 2 adapters, fp16, scale 2."""
    ids = np.array([0, 0, 1, 1], dtype=np.int32)
    return random_problem((1,), n=4, h_in=4096, h_out=4096, r=16, n_adapters=2,
                          dtype=F16, scale=2.0, ids=ids, name="tiny_4tok_2ad")


def decode7b() -> Problem:
    """Llama2-7B decode projection: 32 tokens, 32 distinct adapters (a seeded
    permutation of ids 0..31 over the tokens), h = 4096, r = 16, fp16, scale 32/16."""
    return random_problem((2,), n=32, h_in=4096, h_out=4096, r=16, n_adapters=32,
                          dtype=F16, scale=2.0, id_dist="permutation",
                          name="decode7b_bs32_32ad")


def popularity_sweep(variant: str) -> Problem:
    """7B decode shape, 32 tokens drawn from a pool of 64 adapters, fp16, scale 2:
    (a) identical (one adapter), (b) uniform per token, (c) truncated Zipf s = 1.5."""
    idx = {"a": 0, "b": 1, "c": 2}[variant]
    rng = _streams((3, idx), 6)[5]
    if variant == "a":
        ids = np.zeros(32, dtype=np.int32)
    elif variant == "b":
        ids = rng.integers(0, 64, size=32, dtype=np.int32)
    else:
        ids = truncated_zipf_ids(rng, 32, 64, 1.5)
    name = {"a": "sweep_identical", "b": "sweep_uniform64", "c": "sweep_zipf1.5_64"}[variant]
    return random_problem((3, idx), n=32, h_in=4096, h_out=4096, r=16, n_adapters=64,
                          dtype=F16, scale=2.0, ids=ids, name=name)


PREFILL13B_SHAPES = {"qo": (5120, 5120), "gateup": (5120, 13824), "down": (13824, 5120)}


def prefill13b(proj: str) -> Problem:
    """Llama2-13B prefill: 4 requests x 512 tokens (request-major rows), each request
    on its own adapter (ids a seeded permutation of 0..3), r = 16, bf16, scale 2."""
    h_in, h_out = PREFILL13B_SHAPES[proj]
    idx = list(PREFILL13B_SHAPES).index(proj)
    rng = _streams((4, idx), 6)[5]
    ids = np.repeat(rng.permutation(4).astype(np.int32), 512)
    return random_problem((4, idx), n=2048, h_in=h_in, h_out=h_out, r=16, n_adapters=4,
                          dtype=BF16, scale=2.0, ids=ids, name=f"prefill13b_{proj}")


MIXED70B_SHAPES = {
    "q": (8192, 8192), "k": (8192, 1024), "v": (8192, 1024), "o": (8192, 8192),
    "gate": (8192, 28672), "up": (8192, 28672), "down": (28672, 8192),
}


def mixed70b_ids(rng: np.random.Generator) -> np.ndarray:
    """64 decode tokens over adapters 0..47 (truncated Zipf s = 1.2), then a 1024-token
    prefill chunk on adapter 48 and another on adapter 49."""
    dec = truncated_zipf_ids(rng, 64, 48, 1.2)
    return np.concatenate([dec, np.full(1024, 48, np.int32), np.full(1024, 49, np.int32)])


def mixed70b(proj: str, r: int) -> Problem:
    """Llama2-70B layer, one GPU's share of a mixed batch (n = 2112), bf16,
    r in {16, 64} with scale = 32 / r."""
    assert r in (16, 64)
    h_in, h_out = MIXED70B_SHAPES[proj]
    idx = list(MIXED70B_SHAPES).index(proj)
    rng = _streams((5, 0), 6)[5]            # the same batch for every projection
    ids = mixed70b_ids(rng)
    return random_problem((5, r, idx), n=ids.size, h_in=h_in, h_out=h_out, r=r,
                          n_adapters=50, dtype=BF16, scale=32.0 / r, ids=ids,
                          name=f"mixed70b_r{r}_{proj}")


def decode7b_bs(n: int) -> Problem:
    """The 7B decode projection at batch size n (1..64): n tokens, each on its own adapter
    (a seeded permutation of ids 0..n-1), h = 4096, r = 16, fp16, scale 2."""
    assert 1 <= n <= 64
    return random_problem((6, n), n=n, h_in=4096, h_out=4096, r=16, n_adapters=n,
                          dtype=F16, scale=2.0, id_dist="permutation",
                          name=f"decode7b_bs{n}")


def prefill13b_len(length: int, proj: str = "gateup") -> Problem:
    """The 13B prefill projection with 4 requests of `length` tokens each (request-major
    rows, each request on its own adapter), r = 16, bf16, scale 2."""
    h_in, h_out = PREFILL13B_SHAPES[proj]
    rng = _streams((7, length), 6)[5]
    ids = np.repeat(rng.permutation(4).astype(np.int32), length)
    return random_problem((7, length, h_in), n=4 * length, h_in=h_in, h_out=h_out, r=16,
                          n_adapters=4, dtype=BF16, scale=2.0, ids=ids,
                          name=f"prefill13b_{proj}_len{length}")


@dataclasses.dataclass
class RankedProblem:
    """One mixed-rank call: adapters numbered across ``pools`` (pool k holds ids
    off_k .. off_k + P_k - 1, off_k = sum of the earlier pools' sizes); row t gets
    ``y[t] += scales[r] * (x[t] @ A[ids[t]]) @ B[ids[t]]`` with its adapter's rank r."""

    name: str
    dtype: str
    ids: np.ndarray          # int32 [n]
    x: np.ndarray            # [n, h_in]
    y: np.ndarray            # [n, h_out]
    pools: list              # [(A [P_k, r_k, h_in], B [P_k, h_out, r_k])]
    scales: dict             # rank -> scale

    @property
    def n(self) -> int:
        return int(self.ids.shape[0])

    @property
    def h_in(self) -> int:
        return int(self.x.shape[1])

    @property
    def h_out(self) -> int:
        return int(self.y.shape[1])

    def ranks(self) -> np.ndarray:
        """Rank of every adapter id."""
        return np.concatenate([np.full(A.shape[0], A.shape[1], np.int32) for A, _ in self.pools])


def random_ranked_problem(seed: Sequence[int], *, n: int, h_in: int, h_out: int, pools,
                          dtype: str, ids: Optional[np.ndarray] = None,
                          name: str = "ranked") -> RankedProblem:
    """``pools`` = [(P_k, r_k)]; ids uniform over all adapters unless given; the scale of
    rank r is 32 / r."""
    g_ids, g_x, g_y, g_a, g_b = _streams(seed)
    total = sum(P for P, _ in pools)
    if ids is None:
        ids = g_ids.integers(0, total, size=n, dtype=np.int32)
    x = quantize(_normal(g_x, (n, h_in), 1.0), dtype)
    y = quantize(_normal(g_y, (n, h_out), 1.0), dtype)
    out = []
    for P, r in pools:
        A = quantize(_normal(g_a, (P, r, h_in), 1.0 / np.sqrt(h_in)), dtype)
        B = quantize(_normal(g_b, (P, h_out, r), 1.0 / np.sqrt(r)), dtype)
        out.append((A, B))
    scales = {r: 32.0 / r for _, r in pools}
    return RankedProblem(name, dtype, np.ascontiguousarray(ids, dtype=np.int32), x, y, out, scales)


def mixed70b_ranked(proj: str) -> RankedProblem:
    """The 70B mixed batch with both ranks in one call: of the 50 adapters, the even ones
    (including prefill adapter 48) have r = 16 and the odd ones (including 49) r = 64.
    Pool 0 holds the 25 rank-16 adapters, pool 1 the 25 rank-64 ones; scale 32 / r."""
    h_in, h_out = MIXED70B_SHAPES[proj]
    idx = list(MIXED70B_SHAPES).index(proj)
    orig = mixed70b_ids(_streams((5, 0), 6)[5])
    ids = np.where(orig % 2 == 0, orig // 2, 25 + orig // 2).astype(np.int32)
    return random_ranked_problem((8, idx), n=ids.size, h_in=h_in, h_out=h_out,
                                 pools=[(25, 16), (25, 64)], dtype=BF16, ids=ids,
                                 name=f"mixed70b_rmix_{proj}")


def all_workloads(include_large: bool = True):
    """(name, factory) pairs for every workload projection."""
    out = [("tiny", tiny), ("decode7b", decode7b)]
    out += [(f"sweep_{v}", (lambda v=v: popularity_sweep(v))) for v in "abc"]
    if include_large:
        out += [(f"prefill13b_{p}", (lambda p=p: prefill13b(p))) for p in PREFILL13B_SHAPES]
        out += [(f"mixed70b_r{r}_{p}", (lambda p=p, r=r: mixed70b(p, r)))
                for r in (16, 64) for p in MIXED70B_SHAPES]
    return out


# --------------------------------------------------------------------------------------
# structured inputs for exactness and gather checks
# --------------------------------------------------------------------------------------
def exact_problem(seed: Sequence[int], *, n: int, h_in: int, h_out: int, r: int,
                  n_adapters: int, dtype: str, ids: Optional[np.ndarray] = None,
                  name: str = "exact") -> Problem:
    """Inputs on power-of-two grids so that every product and partial sum of the method
    is exact in float32 whatever the summation order:

    x in {-1, 0, 1};  A in {-1, 0, 1} * 2**-6;  B in {-1, 0, 1} * 2**-2;
    y = k * 2**-8 with |k| <= 255;  scale = 2.

    Then |v| <= h_in * 2**-6 on a 2**-6 grid, the update is on a 2**-7 grid and
    y + update on a 2**-8 grid; for h_in <= 28672 and r <= 64 every intermediate
    needs at most 22 significant bits.  All values are exactly representable in
    fp16 and bf16.
    """
    assert h_in <= 28672 and r <= 64
    g_ids, g_x, g_y, g_a, g_b = _streams(seed)
    if ids is None:
        ids = g_ids.integers(0, n_adapters, size=n, dtype=np.int32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    x = g_x.integers(-1, 2, size=(n, h_in)).astype(np.float32)
    A = g_a.integers(-1, 2, size=(n_adapters, r, h_in)).astype(np.float32) * np.float32(2.0 ** -6)
    B = g_b.integers(-1, 2, size=(n_adapters, h_out, r)).astype(np.float32) * np.float32(0.25)
    y = g_y.integers(-255, 256, size=(n, h_out)).astype(np.float32) * np.float32(2.0 ** -8)
    return Problem(name, dtype, ids, quantize(x, dtype), quantize(y, dtype),
                   quantize(A, dtype), quantize(B, dtype), 2.0)


def gather_probe(seed: Sequence[int], *, n: int, h_in: int, h_out: int, r: int,
                 n_adapters: int, dtype: str, ids: Optional[np.ndarray] = None,
                 name: str = "gather_probe") -> Problem:
    """Adapters that reveal which row and which adapter each output used.

    Column j of adapter a's A selects input column (a*r + j) mod h_in with weight
    2**-6; row j of adapter a's B writes to output column (a*r + j) mod h_out with
    weight 1.  x rows carry integers in [-7, 7], y is zero and scale = 1, so row t's
    update is 2**-6 * x[t, (a*r + j) mod h_in] in output column (a*r + j) mod h_out:
    a wrong row or a wrong adapter moves or changes values.  Every value is exact
    in fp16 and bf16 and every intermediate is exact in float32.
    """
    assert r <= h_in and r <= h_out
    g_ids, g_x, _, _, _ = _streams(seed)
    if ids is None:
        ids = g_ids.integers(0, n_adapters, size=n, dtype=np.int32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    x = g_x.integers(-7, 8, size=(n, h_in)).astype(np.float32)
    A = np.zeros((n_adapters, r, h_in), np.float32)
    B = np.zeros((n_adapters, h_out, r), np.float32)
    for a in range(n_adapters):
        for j in range(r):
            A[a, j, (a * r + j) % h_in] = 2.0 ** -6
            B[a, (a * r + j) % h_out, j] = 1.0
    y = np.zeros((n, h_out), np.float32)
    return Problem(name, dtype, ids, quantize(x, dtype), quantize(y, dtype),
                   quantize(A, dtype), quantize(B, dtype), 1.0)
