"""fp64 CPU oracle for SGMV -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The GPU library never does, and this
module imports nothing from it: the two share no code.  It is plain and slow on
purpose: every function is the definition written out, with numpy as the only
library primitive (a float64 matrix product).

What is computed (Punica pages):

* project overview (vecbase.com), "How It Works": a LoRA model is the pretrained
  weight W plus two smaller matrices A and B, applied through SGMV;
* paper summary (research.elamur.ai), "Summary": in one batch the backbone runs as
  one ordinary GEMM and the per-adapter low-rank additions are computed together,
  requests for the same adapter grouped;
* same page, "Interesting ideas", I2: the batch is sorted by adapter so that rows of
  one adapter form a contiguous segment.

Grouping is a reordering only, so the result of SGMV is, row by row,

    y_out[t, :] = y_in[t, :] + scale * (x[t, :] @ A[a_t]) @ B[a_t],   a_t = ids[t]

with A of shape h_in x r and B of shape r x h_out.  The oracle evaluates exactly this
in float64 from the exactly decoded fp16/bf16 inputs and does not round the result.
The pages give no layout, scale or precision; the readings taken here:

* the update is ``scale * ((x @ A) @ B)`` with the scale applied to the product;
* storage (shared with the input generator): ``A_pool[a]`` is ``[r, h_in]`` (row j is
  column j of A) and ``B_pool[a]`` is ``[h_out, r]`` (row c is column c of B);
* the segment table is a *stable* sort by adapter id: ties keep caller order,
  segments appear in ascending adapter id, adapters with no rows make no segment;
* the pages fix no rank and no scale per adapter.  For a batch whose adapters have
  different ranks, every row uses its own adapter's A, B and rank, and each rank has
  its own scale (LoRA scales are usually alpha / r); rows are grouped by rank first,
  then by adapter.

Every function here is pinned by tests that do not reuse its code: exact rational
brute force on tiny inputs, a hand-worked example, a closed form, invariants, and
the exactness of power-of-two-grid inputs.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

F16 = "f16"
BF16 = "bf16"


# --------------------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------------------
def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of fp16 (numpy.float16) or bf16 (uint16 bits) storage."""
    if dtype == F16:
        assert a.dtype == np.float16
        return a.astype(np.float64)
    if dtype == BF16:
        assert a.dtype == np.uint16
        bits32 = a.astype(np.uint32) << np.uint32(16)
        return bits32.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_io(v: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once, to nearest with ties to even, into the I/O format.

    fp16 uses numpy's direct double -> half conversion (correctly rounded).  bf16 is
    done here from the definition: a normal bfloat16 keeps 8 significant bits, so
    with v = m * 2**e (0.5 <= |m| < 1) the result is rint(m * 2**8) * 2**(e - 8),
    rint being round-half-even.  Only finite values within bfloat16's normal range
    (or zero) are accepted.
    """
    v = np.asarray(v, dtype=np.float64)
    if dtype == F16:
        return v.astype(np.float16)
    if dtype == BF16:
        m, e = np.frexp(v)
        nz = v != 0
        assert np.all(np.isfinite(v))
        assert np.all(np.abs(v[nz]) >= 2.0 ** -126) and np.all(np.abs(v) < 2.0 ** 127)
        q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
        bits = q.astype(np.float32).view(np.uint32) >> np.uint32(16)
        return bits.astype(np.uint16)
    raise ValueError(dtype)


# --------------------------------------------------------------------------------------
# segment metadata (the paper summary's idea I2: sort the batch by adapter)
# --------------------------------------------------------------------------------------
def segments(ids: np.ndarray, n_adapters: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Stable counting sort of the caller's rows by adapter id.

    Returns ``perm`` (int32[n]: caller row at sorted position i), ``seg_starts``
    (int32[S+1]: the sorted rows of segment s are seg_starts[s] .. seg_starts[s+1]-1)
    and ``seg_adapter`` (int32[S]: the adapter of segment s), S being the number of
    distinct ids.  Written with plain Python loops.
    """
    ids = [int(t) for t in np.asarray(ids).reshape(-1)]
    for t in ids:
        if not 0 <= t < n_adapters:
            raise ValueError(f"adapter id {t} outside [0, {n_adapters})")
    count = [0] * n_adapters
    for t in ids:
        count[t] += 1
    start = [0] * n_adapters          # exclusive prefix sum of the counts
    acc = 0
    for a in range(n_adapters):
        start[a] = acc
        acc += count[a]
    perm = [0] * len(ids)
    fill = list(start)
    for i, t in enumerate(ids):       # caller order -> stable
        perm[fill[t]] = i
        fill[t] += 1
    seg_starts, seg_adapter = [], []
    for a in range(n_adapters):
        if count[a]:
            seg_starts.append(start[a])
            seg_adapter.append(a)
    seg_starts.append(len(ids))
    return (np.array(perm, dtype=np.int32), np.array(seg_starts, dtype=np.int32),
            np.array(seg_adapter, dtype=np.int32))


def ptr_table(adapter_base: np.ndarray, seg_adapter: np.ndarray) -> np.ndarray:
    """Per-segment pointer table: entry s is the base address of segment s's adapter."""
    base = np.asarray(adapter_base, dtype=np.uint64)
    return np.array([base[int(a)] for a in seg_adapter], dtype=np.uint64)


# --------------------------------------------------------------------------------------
# the low-rank update
# --------------------------------------------------------------------------------------
class DecodedPool:
    """Adapter pool in storage format, decoded to float64 one adapter at a time, on first
    use (each decoded adapter is kept).  ``shape`` is the storage pool's shape."""

    def __init__(self, pool: np.ndarray, dtype: str):
        self.pool, self.dtype, self.shape = pool, dtype, pool.shape
        self._done = {}

    def __getitem__(self, a: int) -> np.ndarray:
        if a not in self._done:
            self._done[a] = decode(self.pool[a], self.dtype)
        return self._done[a]


def shrink_f64(X: np.ndarray, ids: np.ndarray, A64) -> np.ndarray:
    """v[t, :] = X[t, :] @ A[ids[t]] on float64 values: X [n, h_in]; A64[a] is adapter
    a's stored A, [r, h_in] (column j of A is row j), and A64.shape[1] is r."""
    n, r = X.shape[0], A64.shape[1]
    v = np.zeros((n, r), dtype=np.float64)
    for a in np.unique(ids):
        rows = np.nonzero(ids == a)[0]
        A_a = A64[int(a)]
        v[rows] = X[rows] @ A_a.T
    return v


def expand_f64(Y: np.ndarray, v: np.ndarray, ids: np.ndarray, B64, scale: float) -> np.ndarray:
    """Y[t, :] + scale * (v[t, :] @ B[ids[t]]) on float64 values: B64[a] is adapter a's
    stored B, [h_out, r] (column c of B is row c)."""
    out = Y.copy()
    for a in np.unique(ids):
        rows = np.nonzero(ids == a)[0]
        B_a = B64[int(a)]
        out[rows] += float(scale) * (np.asarray(v, np.float64)[rows] @ B_a.T)
    return out


def shrink(x: np.ndarray, ids: np.ndarray, A_pool: np.ndarray, dtype: str) -> np.ndarray:
    """v[t, :] = x[t, :] @ A[ids[t]]  in float64, caller row order, shape [n, r]."""
    return shrink_f64(decode(x, dtype), ids, DecodedPool(A_pool, dtype))


def expand(y: np.ndarray, v: np.ndarray, ids: np.ndarray, B_pool: np.ndarray,
           scale: float, dtype: str) -> np.ndarray:
    """y_in[t, :] + scale * (v[t, :] @ B[ids[t]])  in float64 (not rounded)."""
    return expand_f64(decode(y, dtype), v, ids, DecodedPool(B_pool, dtype), scale)


def lora_add_f64(Y: np.ndarray, X: np.ndarray, ids: np.ndarray, A64, B64,
                 scale: float) -> np.ndarray:
    """SGMV on float64 values (see shrink_f64 / expand_f64)."""
    return expand_f64(Y, shrink_f64(X, ids, A64), ids, B64, scale)


def lora_add(y: np.ndarray, x: np.ndarray, ids: np.ndarray, A_pool: np.ndarray,
             B_pool: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """SGMV result: y_in + scale * (x @ A[a_t]) @ B[a_t] per row, float64, unrounded."""
    return lora_add_f64(decode(y, dtype), decode(x, dtype), ids, DecodedPool(A_pool, dtype),
                        DecodedPool(B_pool, dtype), scale)


def lora_add_problem(p) -> np.ndarray:
    """``lora_add`` on a ``workloads.Problem``."""
    return lora_add(p.y, p.x, p.ids, p.A, p.B, p.scale, p.dtype)


# --------------------------------------------------------------------------------------
# mixed ranks: adapters of several ranks in one call
# --------------------------------------------------------------------------------------
def segments_ranked(ids: np.ndarray, adapter_rank: np.ndarray):
    """Stable sort of the caller's rows by (rank of the row's adapter, adapter id): the
    batch sorted by adapter (paper summary, "Interesting ideas", I2) with the rank as the
    leading key.  Returns (perm, [(r, row0, n, seg_starts relative to row0, seg_adapter)]
    for every rank present, ascending r)."""
    ids = np.asarray(ids, dtype=np.int64)
    rank = np.asarray(adapter_rank, dtype=np.int64)
    keys = [(int(rank[a]), int(a), t) for t, a in enumerate(ids)]
    keys.sort()
    perm = np.array([k[2] for k in keys], dtype=np.int32)
    groups = []
    for r in sorted(set(int(rank[a]) for a in ids)):
        pos = [i for i, k in enumerate(keys) if k[0] == r]
        row0, n = pos[0], len(pos)
        starts, seg_ad = [], []
        for i in pos:
            a = keys[i][1]
            if not seg_ad or seg_ad[-1] != a:
                starts.append(i - row0)
                seg_ad.append(a)
        starts.append(n)
        groups.append((r, row0, n, np.array(starts, np.int32), np.array(seg_ad, np.int32)))
    return perm, groups


def lora_add_ranked(y: np.ndarray, x: np.ndarray, ids: np.ndarray, pools, scales,
                    dtype: str) -> np.ndarray:
    """Mixed ranks: ``pools`` is a list of (A_pool [P_k, r_k, h_in], B_pool [P_k, h_out, r_k])
    whose adapters are numbered one after another (pool k holds ids off_k .. off_k+P_k-1),
    and ``scales[r]`` is the scale of rank r.  Row t gets
    y_in[t] + scales[r] * (x[t] @ A[ids[t]]) @ B[ids[t]] with its adapter's own rank r;
    float64, unrounded."""
    ids = np.asarray(ids)
    out = decode(y, dtype).copy()
    off = 0
    for A_k, B_k in pools:
        P, r = int(A_k.shape[0]), int(A_k.shape[1])
        rows = np.nonzero((ids >= off) & (ids < off + P))[0]
        if rows.size:
            local = (ids[rows] - off).astype(np.int32)
            v = shrink(x[rows], local, A_k, dtype)
            out[rows] = expand(y[rows], v, local, B_k, scales[r], dtype)
        off += P
    return out
