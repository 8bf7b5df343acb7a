"""Python binding of libsgmv (SGMV: segmented gather matrix-vector multiplication).

Two layers, both argument marshalling only -- every step of the computation runs in
libsgmv's HIP kernels or its C++ segment builder:

* ``sgmv_*`` functions mirror the C ABI one to one (raw device addresses as ints,
  host arrays as numpy);
* ``Batch`` / ``lora_add`` / ``shrink`` / ``expand`` take torch tensors: PyTorch only
  provides device memory and the current HIP stream.

Layouts (see include/sgmv.h): x [n, h_in], y [n, h_out] row-major; an adapter pool
``A_pool`` [P, r, h_in] (row j of A[a] is column j of the h_in x r matrix) and
``B_pool`` [P, h_out, r] (row c is column c of the r x h_out matrix).
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Sequence, Union

import numpy as np

from . import _lib
from ._lib import BF16, F16, SgmvError, check  # noqa: F401


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


# --------------------------------------------------------------------------------------
# C ABI mirror
# --------------------------------------------------------------------------------------
def sgmv_abi_version() -> int:
    return int(_lib.lib().sgmv_abi_version())


def sgmv_status_string(status: int) -> str:
    return _lib.status_string(status)


@dataclasses.dataclass
class SegmentTable:
    """Host segment metadata of one batch (see sgmv_build_segments)."""
    perm: np.ndarray          # int32 [n]
    seg_starts: np.ndarray    # int32 [S+1]
    seg_adapter: np.ndarray   # int32 [S]
    n_segments: int
    min_seg_len: int
    max_seg_len: int

    @property
    def n(self) -> int:
        return int(self.perm.shape[0])


def sgmv_build_segments(adapter_ids, n_adapters: int) -> SegmentTable:
    ids = np.ascontiguousarray(adapter_ids, dtype=np.int32)
    n = int(ids.shape[0])
    # perm [n] | seg_starts [n+1] | seg_adapter [n] | n_segments, min, max: one buffer, so
    # that numpy's (slow) ctypes address is taken once
    buf = np.empty(3 * n + 4, np.int32)
    a = buf.ctypes.data
    st = _lib.lib().sgmv_build_segments(_ptr(ids), n, int(n_adapters), a, a + 4 * n,
                                        a + 4 * (2 * n + 1), a + 4 * (3 * n + 1),
                                        a + 4 * (3 * n + 2), a + 4 * (3 * n + 3))
    check(st, "sgmv_build_segments")
    s, lo, hi = (int(v) for v in buf[3 * n + 1:])
    return SegmentTable(buf[:n], buf[n: n + s + 1], buf[2 * n + 1: 2 * n + 1 + s], s, lo, hi)


def sgmv_build_ptr_table(adapter_base, seg_adapter) -> np.ndarray:
    base = np.ascontiguousarray(adapter_base, dtype=np.uint64)
    seg_ad = np.ascontiguousarray(seg_adapter, dtype=np.int32)
    out = np.empty(max(seg_ad.shape[0], 1), np.uint64)
    st = _lib.lib().sgmv_build_ptr_table(_ptr(base), int(base.shape[0]), _ptr(seg_ad),
                                         int(seg_ad.shape[0]), _ptr(out))
    check(st, "sgmv_build_ptr_table")
    return out[: seg_ad.shape[0]]


def sgmv_workspace_bytes(n: int, h_in: int, r: int) -> int:
    return int(_lib.lib().sgmv_workspace_bytes(int(n), int(h_in), int(r)))


def sgmv_check_workspace(stream, workspace, flags, clear) -> int:
    return _lib.lib().sgmv_check_workspace(stream, workspace, flags, int(clear))


def workspace_flags(workspace, clear: bool = False, stream=None) -> int:
    """The workspace's device-side flag bits (FLAG_* in ``_lib``), read after every call
    enqueued on ``stream`` has finished; ``clear`` resets them to zero."""
    f = np.zeros(1, np.int32)
    st = sgmv_check_workspace(_stream_handle(stream), workspace.data_ptr(), _ptr(f), clear)
    if st not in (_lib.OK, _lib.ERR_DEVICE):
        check(st, "sgmv_check_workspace")
    return int(f[0])


def sgmv_shrink(stream, dtype, v, x, ld_x, A_ptrs, seg_starts, perm, n, n_segments,
                min_seg_len, max_seg_len, h_in, r, workspace, workspace_bytes) -> int:
    return _lib.lib().sgmv_shrink(stream, dtype, v, x, ld_x, A_ptrs, seg_starts, perm, n,
                                  n_segments, min_seg_len, max_seg_len, h_in, r, workspace,
                                  workspace_bytes)


def sgmv_expand(stream, dtype, y, ld_y, v, B_ptrs, seg_starts, perm, n, n_segments,
                min_seg_len, max_seg_len, r, h_out, scale) -> int:
    return _lib.lib().sgmv_expand(stream, dtype, y, ld_y, v, B_ptrs, seg_starts, perm, n,
                                  n_segments, min_seg_len, max_seg_len, r, h_out, float(scale))


def sgmv_lora_add(stream, dtype, y, ld_y, x, ld_x, A_ptrs, B_ptrs, seg_starts, perm, n,
                  n_segments, min_seg_len, max_seg_len, h_in, h_out, r, scale, workspace,
                  workspace_bytes) -> int:
    return _lib.lib().sgmv_lora_add(stream, dtype, y, ld_y, x, ld_x, A_ptrs, B_ptrs, seg_starts,
                                    perm, n, n_segments, min_seg_len, max_seg_len, h_in, h_out, r,
                                    float(scale), workspace, workspace_bytes)


# --------------------------------------------------------------------------------------
# torch layer
# --------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float16 or bfloat16)")


def as_tensor(arr: np.ndarray, dtype: str, device=None):
    """Storage array of the input generator ("f16": float16, "bf16": uint16 bits) as a
    torch tensor of the matching dtype (no value conversion)."""
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if dtype == "f16":
        t = torch.from_numpy(a.view(np.float16))
    elif dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        raise ValueError(dtype)
    return t.to(device) if device is not None else t


def adapter_bases(pool) -> np.ndarray:
    """Device address of each adapter in a pool tensor [P, ...] or a list of tensors."""
    if isinstance(pool, (list, tuple)):
        return np.array([int(t.data_ptr()) for t in pool], dtype=np.uint64)
    stride = pool.stride(0) * pool.element_size()
    return np.uint64(pool.data_ptr()) + np.arange(pool.shape[0], dtype=np.uint64) * np.uint64(stride)


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


@dataclasses.dataclass
class Batch:
    """Segment metadata of one batch, resident on the device (one H2D copy).

    ``table`` is the host SegmentTable; ``dev`` holds [A_ptrs | B_ptrs | seg_starts |
    perm] in one device buffer, and the ``*_addr`` fields are device addresses into it.
    """
    table: SegmentTable
    n_adapters: int
    rank: int
    h_in: int
    h_out: int
    dev: object
    A_ptrs_addr: int
    B_ptrs_addr: int
    seg_starts_addr: int
    perm_addr: int

    @property
    def n(self) -> int:
        return self.table.n

    @classmethod
    def build(cls, adapter_ids, A_pool, B_pool, device=None, identity_perm: bool = False):
        """Sort ``adapter_ids`` (host) into segments and upload the tables.

        ``A_pool`` / ``B_pool`` are pool tensors [P, ...] or lists of per-adapter tensors
        on the device.  ``identity_perm`` passes perm = NULL (rows already sorted)."""
        torch = _torch()
        if isinstance(A_pool, (list, tuple)):
            n_adapters, rank = len(A_pool), int(A_pool[0].shape[0])
            h_in, h_out = int(A_pool[0].shape[1]), int(B_pool[0].shape[0])
            As, Bs = list(A_pool), list(B_pool)
        else:
            n_adapters, rank = int(A_pool.shape[0]), int(A_pool.shape[1])
            h_in, h_out = int(A_pool.shape[2]), int(B_pool.shape[1])
            As, Bs = [A_pool[0]], [B_pool[0]]
        _check_adapters(As, Bs, rank, h_in, h_out, n_adapters, len(B_pool))
        tab = sgmv_build_segments(adapter_ids, n_adapters)
        if identity_perm and not np.array_equal(tab.perm, np.arange(tab.n, dtype=np.int32)):
            raise ValueError("identity_perm requires adapter_ids to be sorted")
        a_ptr = sgmv_build_ptr_table(adapter_bases(A_pool), tab.seg_adapter)
        b_ptr = sgmv_build_ptr_table(adapter_bases(B_pool), tab.seg_adapter)
        buf = cls.pack(tab, a_ptr, b_ptr)
        if device is None:
            device = A_pool[0].device if isinstance(A_pool, (list, tuple)) else A_pool.device
        dev = torch.from_numpy(buf).to(device)
        base = int(dev.data_ptr())
        S, n = tab.n_segments, tab.n
        off_b = 8 * S
        off_s = 16 * S
        off_p = off_s + 4 * (S + 1)
        return cls(tab, n_adapters, rank, h_in, h_out, dev, base, base + off_b, base + off_s,
                   0 if identity_perm else base + off_p)

    @staticmethod
    def pack(tab: SegmentTable, a_ptr: np.ndarray, b_ptr: np.ndarray) -> np.ndarray:
        S, n = tab.n_segments, tab.n
        nbytes = 16 * S + 4 * (S + 1) + 4 * n
        buf = np.zeros(max(nbytes, 16), np.uint8)
        buf[: 8 * S] = a_ptr.view(np.uint8)
        buf[8 * S: 16 * S] = b_ptr.view(np.uint8)
        buf[16 * S: 16 * S + 4 * (S + 1)] = tab.seg_starts.view(np.uint8)
        buf[16 * S + 4 * (S + 1): nbytes] = tab.perm.view(np.uint8)
        return buf


def _check_adapters(As, Bs, r: int, h_in: int, h_out: int, n_a: int, n_b: int):
    """Every adapter's A is a dense [r, h_in] and B a dense [h_out, r] array (the kernels
    read them with these strides)."""
    if n_a != n_b:
        raise ValueError("A and B pools hold different numbers of adapters")
    for A, B in zip(As, Bs):
        if tuple(A.shape[-2:]) != (r, h_in) or tuple(B.shape[-2:]) != (h_out, r):
            raise ValueError(f"adapter shapes {tuple(A.shape)} / {tuple(B.shape)} do not match "
                             f"A [{r}, {h_in}] and B [{h_out}, {r}]")
        if A.stride(-1) != 1 or A.stride(-2) != h_in or B.stride(-1) != 1 or B.stride(-2) != r:
            raise ValueError("each adapter's A and B must be dense row-major arrays")


def _check_io(x, y, h_in: int, h_out: int):
    if x.shape[1] != h_in or y.shape[1] != h_out:
        raise ValueError(f"x [n, {x.shape[1]}] / y [n, {y.shape[1]}] do not match the adapters' "
                         f"h_in = {h_in}, h_out = {h_out}")


def make_workspace(n: int, h_in: int, r: int, device):
    """Zero-filled, 256-byte aligned workspace for shrink / lora_add."""
    torch = _torch()
    nbytes = sgmv_workspace_bytes(n, h_in, r)
    if nbytes == 0:
        raise ValueError("invalid sizes for sgmv_workspace_bytes")
    ws = torch.zeros(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-int(ws.data_ptr())) % 256
    return ws[off: off + nbytes]


def _check_rows(t, n: int, name: str):
    if t.dim() != 2 or t.shape[0] != n or t.stride(1) != 1:
        raise ValueError(f"{name} must be [n, h] with unit column stride")


def lora_add(y, x, batch: Batch, scale: float, workspace=None, stream=None):
    """y[t] += scale * (x[t] @ A[a_t]) @ B[a_t] in place (fused shrink + expand)."""
    n = batch.n
    _check_rows(x, n, "x")
    _check_rows(y, n, "y")
    if x.dtype != y.dtype:
        raise TypeError("x and y must share a dtype")
    _check_io(x, y, batch.h_in, batch.h_out)
    r = _infer_rank(batch)
    if workspace is None:
        workspace = make_workspace(n, x.shape[1], r, x.device)
    t = batch.table
    st = sgmv_lora_add(_stream_handle(stream), dtype_code(y), y.data_ptr(), y.stride(0),
                       x.data_ptr(), x.stride(0), batch.A_ptrs_addr, batch.B_ptrs_addr,
                       batch.seg_starts_addr, batch.perm_addr or None, n, t.n_segments,
                       t.min_seg_len, t.max_seg_len, x.shape[1], y.shape[1], r, scale,
                       workspace.data_ptr(), workspace.numel())
    check(st, "sgmv_lora_add")
    return y


def shrink(x, batch: Batch, r: Optional[int] = None, workspace=None, stream=None):
    """v[i] = x[perm[i]] @ A[segment of i] as float32 [n, r] in sorted order."""
    torch = _torch()
    n = batch.n
    _check_rows(x, n, "x")
    if x.shape[1] != batch.h_in:
        raise ValueError(f"x [n, {x.shape[1]}] does not match the adapters' h_in = {batch.h_in}")
    r = r or _infer_rank(batch)
    v = torch.empty((n, r), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = make_workspace(n, x.shape[1], r, x.device)
    t = batch.table
    st = sgmv_shrink(_stream_handle(stream), dtype_code(x), v.data_ptr(), x.data_ptr(),
                     x.stride(0), batch.A_ptrs_addr, batch.seg_starts_addr,
                     batch.perm_addr or None, n, t.n_segments, t.min_seg_len, t.max_seg_len,
                     x.shape[1], r, workspace.data_ptr(), workspace.numel())
    check(st, "sgmv_shrink")
    return v


def expand(y, v, batch: Batch, scale: float, stream=None):
    """y[perm[i]] += scale * v[i] @ B[segment of i] in place."""
    n = batch.n
    _check_rows(y, n, "y")
    if y.shape[1] != batch.h_out or tuple(v.shape) != (n, batch.rank):
        raise ValueError("y or v does not match the batch's h_out and rank")
    t = batch.table
    st = sgmv_expand(_stream_handle(stream), dtype_code(y), y.data_ptr(), y.stride(0),
                     v.data_ptr(), batch.B_ptrs_addr, batch.seg_starts_addr,
                     batch.perm_addr or None, n, t.n_segments, t.min_seg_len, t.max_seg_len,
                     v.shape[1], y.shape[1], scale)
    check(st, "sgmv_expand")
    return y


def _infer_rank(batch: Batch) -> int:
    return int(batch.rank)


# --------------------------------------------------------------------------------------
# mixed ranks: adapters of ranks 16, 32 and 64 in one call
# --------------------------------------------------------------------------------------
@dataclasses.dataclass
class RankedTable:
    """Host segment metadata of a mixed-rank batch (see sgmv_build_segments_ranked)."""
    perm: np.ndarray          # int32 [n]
    seg_starts: np.ndarray    # int32 [S + G]: per group, starts relative to its row0
    seg_adapter: np.ndarray   # int32 [S]
    groups: list              # [_lib.RankGroup], ascending r

    @property
    def n(self) -> int:
        return int(self.perm.shape[0])

    @property
    def n_segments(self) -> int:
        return int(self.seg_adapter.shape[0])


def sgmv_build_segments_ranked(adapter_ids, adapter_rank) -> RankedTable:
    ids = np.ascontiguousarray(np.asarray(adapter_ids), dtype=np.int32)
    rank = np.ascontiguousarray(np.asarray(adapter_rank), dtype=np.int32)
    n = int(ids.shape[0])
    perm = np.zeros(max(n, 1), np.int32)
    starts = np.zeros(n + 3, np.int32)
    seg_ad = np.zeros(max(n, 1), np.int32)
    groups = (_lib.RankGroup * 3)()
    G = np.zeros(1, np.int32)
    st = _lib.lib().sgmv_build_segments_ranked(_ptr(ids), n, int(rank.shape[0]), _ptr(rank),
                                               _ptr(perm), _ptr(starts), _ptr(seg_ad),
                                               ctypes.addressof(groups), _ptr(G))
    check(st, "sgmv_build_segments_ranked")
    gs = [groups[i] for i in range(int(G[0]))]
    S = sum(g.n_segments for g in gs)
    return RankedTable(perm[:n].copy(), starts[: S + len(gs)].copy(), seg_ad[:S].copy(), gs)


def sgmv_lora_add_ranked(stream, dtype, y, ld_y, x, ld_x, A_ptrs, B_ptrs, seg_starts, perm, n,
                         groups, n_groups, h_in, h_out, workspace, workspace_bytes) -> int:
    return _lib.lib().sgmv_lora_add_ranked(stream, dtype, y, ld_y, x, ld_x, A_ptrs, B_ptrs,
                                           seg_starts, perm, n, groups, n_groups, h_in, h_out,
                                           workspace, workspace_bytes)


@dataclasses.dataclass
class RankedBatch:
    """Segment metadata of a mixed-rank batch on the device.  Adapter ids index the
    concatenation of the pools: pool k holds ids offset_k .. offset_k + P_k - 1."""
    table: RankedTable
    h_in: int
    h_out: int
    dev: object
    A_ptrs_addr: int
    B_ptrs_addr: int
    seg_starts_addr: int
    perm_addr: int

    @property
    def n(self) -> int:
        return self.table.n

    @property
    def max_rank(self) -> int:
        return max((g.r for g in self.table.groups), default=16)

    @classmethod
    def build(cls, adapter_ids, pools):
        """``pools`` is a list of (A_pool [P_k, r_k, h_in], B_pool [P_k, h_out, r_k]) device
        tensors."""
        torch = _torch()
        h_in, h_out = int(pools[0][0].shape[2]), int(pools[0][1].shape[1])
        for A, B in pools:
            _check_adapters([A[0]], [B[0]], int(A.shape[1]), h_in, h_out, int(A.shape[0]),
                            int(B.shape[0]))
        rank = np.concatenate([np.full(int(A.shape[0]), int(A.shape[1]), np.int32)
                               for A, _ in pools])
        tab = sgmv_build_segments_ranked(adapter_ids, rank)
        a_base = np.concatenate([adapter_bases(A) for A, _ in pools])
        b_base = np.concatenate([adapter_bases(B) for _, B in pools])
        a_ptr = sgmv_build_ptr_table(a_base, tab.seg_adapter)
        b_ptr = sgmv_build_ptr_table(b_base, tab.seg_adapter)
        S, n = tab.n_segments, tab.n
        ns = int(tab.seg_starts.shape[0])
        nbytes = 16 * S + 4 * ns + 4 * n
        buf = np.zeros(max(nbytes, 16), np.uint8)
        buf[: 8 * S] = a_ptr[:S].view(np.uint8)
        buf[8 * S: 16 * S] = b_ptr[:S].view(np.uint8)
        buf[16 * S: 16 * S + 4 * ns] = tab.seg_starts.view(np.uint8)
        buf[16 * S + 4 * ns: nbytes] = tab.perm.view(np.uint8)
        dev = torch.from_numpy(buf).to(pools[0][0].device)
        base = int(dev.data_ptr())
        return cls(tab, h_in, h_out, dev, base, base + 8 * S, base + 16 * S,
                   base + 16 * S + 4 * ns)


def lora_add_ranked(y, x, batch: RankedBatch, scales, workspace=None, stream=None):
    """y[t] += scale_r * (x[t] @ A[a_t]) @ B[a_t] in place, where r is the rank of a_t's
    pool and ``scales`` maps each rank to its scale."""
    n = batch.n
    _check_rows(x, n, "x")
    _check_rows(y, n, "y")
    if x.dtype != y.dtype:
        raise TypeError("x and y must share a dtype")
    _check_io(x, y, batch.h_in, batch.h_out)
    gs = batch.table.groups
    arr = (_lib.RankGroup * max(len(gs), 1))()
    for i, g in enumerate(gs):
        arr[i] = g
        arr[i].scale = float(scales[g.r])
    if workspace is None:
        workspace = make_workspace(n, x.shape[1], batch.max_rank, x.device)
    st = sgmv_lora_add_ranked(_stream_handle(stream), dtype_code(y), y.data_ptr(), y.stride(0),
                              x.data_ptr(), x.stride(0), batch.A_ptrs_addr, batch.B_ptrs_addr,
                              batch.seg_starts_addr, batch.perm_addr, n, ctypes.addressof(arr),
                              len(gs), x.shape[1], y.shape[1], workspace.data_ptr(),
                              workspace.numel())
    check(st, "sgmv_lora_add_ranked")
    return y


# --------------------------------------------------------------------------------------
# decode path: device-resident adapter ids, adapters in pools, one launch per call
# --------------------------------------------------------------------------------------
def sgmv_build_segments_device(stream, adapter_ids, n, n_adapters, perm, seg_starts,
                               seg_adapter, n_segments) -> int:
    return _lib.lib().sgmv_build_segments_device(stream, adapter_ids, n, n_adapters, perm,
                                                 seg_starts, seg_adapter, n_segments)


def sgmv_lora_add_pool(stream, dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride,
                       B_pool, B_stride, n_adapters, h_in, h_out, r, scale, workspace,
                       workspace_bytes) -> int:
    return _lib.lib().sgmv_lora_add_pool(stream, dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool,
                                         A_stride, B_pool, B_stride, n_adapters, h_in, h_out, r,
                                         float(scale), workspace, workspace_bytes)


def sgmv_lora_add_host_ids(stream, dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool, A_stride,
                           B_pool, B_stride, n_adapters, h_in, h_out, r, scale, workspace,
                           workspace_bytes) -> int:
    """``adapter_ids`` is a HOST address (int32[n], n <= 64)."""
    return _lib.lib().sgmv_lora_add_host_ids(stream, dtype, y, ld_y, x, ld_x, adapter_ids, n,
                                             A_pool, A_stride, B_pool, B_stride, n_adapters,
                                             h_in, h_out, r, float(scale), workspace,
                                             workspace_bytes)


DECODE_MAX_TOKENS = 64   # one-launch decode kernel
POOL_MAX_TOKENS = 4096   # device-side segment sort, then the table kernels


def build_segments_device(ids, n_adapters: int, stream=None):
    """Device segment tables for device int32 ids (n <= 4096): (perm, seg_starts,
    seg_adapter, n_segments) as int32 tensors; n_segments[0] is -1 if an id is out of
    range."""
    torch = _torch()
    n = int(ids.shape[0])
    dev = ids.device
    perm = torch.full((max(n, 1),), -1, dtype=torch.int32, device=dev)
    starts = torch.full((n + 1,), -1, dtype=torch.int32, device=dev)
    seg_ad = torch.full((max(n, 1),), -1, dtype=torch.int32, device=dev)
    S = torch.zeros(1, dtype=torch.int32, device=dev)
    st = sgmv_build_segments_device(_stream_handle(stream), ids.data_ptr(), n, int(n_adapters),
                                    perm.data_ptr(), starts.data_ptr(), seg_ad.data_ptr(),
                                    S.data_ptr())
    check(st, "sgmv_build_segments_device")
    return perm, starts, seg_ad, S


def _layer_pools(A_pool, B_pool, layer):
    """Stacked multi-layer pools [layers, P, ...]: layer ``layer``'s pools (a pointer
    offset of layer * P adapters); 3-D pools are returned as they are."""
    if A_pool.dim() == 4 or B_pool.dim() == 4:
        if layer is None or A_pool.dim() != 4 or B_pool.dim() != 4:
            raise ValueError("stacked [layers, P, ...] pools need a layer index (both pools)")
        return A_pool[layer], B_pool[layer]
    if layer not in (None, 0):
        raise ValueError("a layer index needs stacked [layers, P, ...] pools")
    return A_pool, B_pool


def lora_add_pool(y, x, ids, A_pool, B_pool, scale: float, workspace=None, stream=None,
                  layer: Optional[int] = None):
    """y[t] += scale * (x[t] @ A_pool[ids[t]]) @ B_pool[ids[t]] with device ids (n <= 4096):
    one launch for n <= 64, device segment sort plus the table kernels above.

    ``ids`` is a device int32 tensor [n]; ``A_pool`` [P, r, h_in] and ``B_pool``
    [P, h_out, r] are device tensors with contiguous adapters, or stacked multi-layer
    pools [layers, P, ...] with ``layer`` naming the layer."""
    A_pool, B_pool = _layer_pools(A_pool, B_pool, layer)
    n = int(x.shape[0])
    _check_rows(x, n, "x")
    _check_rows(y, n, "y")
    r = int(A_pool.shape[1])
    _check_adapters([A_pool[0]], [B_pool[0]], r, int(x.shape[1]), int(y.shape[1]),
                    int(A_pool.shape[0]), int(B_pool.shape[0]))
    if ids.dtype != _torch().int32 or ids.dim() != 1 or int(ids.shape[0]) != n:
        raise ValueError("ids must be a device int32 tensor [n]")
    if workspace is None:
        workspace = make_workspace(n, x.shape[1], r, x.device)
    st = sgmv_lora_add_pool(_stream_handle(stream), dtype_code(y), y.data_ptr(), y.stride(0),
                            x.data_ptr(), x.stride(0), ids.data_ptr(), n, A_pool.data_ptr(),
                            A_pool.stride(0), B_pool.data_ptr(), B_pool.stride(0),
                            int(A_pool.shape[0]), x.shape[1], y.shape[1], r, scale,
                            workspace.data_ptr(), workspace.numel())
    check(st, "sgmv_lora_add_pool")
    return y


def lora_add_host_ids(y, x, ids, A_pool, B_pool, scale: float, workspace=None, stream=None,
                      layer: Optional[int] = None):
    """y[t] += scale * (x[t] @ A_pool[ids[t]]) @ B_pool[ids[t]] for a decode batch (n <= 64)
    whose adapter ids are on the host: one launch, the ids travel in its kernel arguments.

    ``ids`` is a host int32 array or CPU tensor [n]; the pools are as for lora_add_pool."""
    A_pool, B_pool = _layer_pools(A_pool, B_pool, layer)
    ids_np = np.ascontiguousarray(
        ids.numpy() if hasattr(ids, "numpy") else np.asarray(ids), dtype=np.int32)
    n = int(x.shape[0])
    _check_rows(x, n, "x")
    _check_rows(y, n, "y")
    if ids_np.ndim != 1 or ids_np.shape[0] != n:
        raise ValueError("ids must be a host int32 array [n]")
    r = int(A_pool.shape[1])
    _check_adapters([A_pool[0]], [B_pool[0]], r, int(x.shape[1]), int(y.shape[1]),
                    int(A_pool.shape[0]), int(B_pool.shape[0]))
    if workspace is None:
        workspace = make_workspace(n, x.shape[1], r, x.device)
    st = sgmv_lora_add_host_ids(_stream_handle(stream), dtype_code(y), y.data_ptr(), y.stride(0),
                                x.data_ptr(), x.stride(0), _ptr(ids_np), n, A_pool.data_ptr(),
                                A_pool.stride(0), B_pool.data_ptr(), B_pool.stride(0),
                                int(A_pool.shape[0]), x.shape[1], y.shape[1], r, scale,
                                workspace.data_ptr(), workspace.numel())
    check(st, "sgmv_lora_add_host_ids")
    return y


def sgmv_lora_add_host_ids_noalloc(stream, dtype, y, ld_y, x, ld_x, adapter_ids, n, A_pool,
                                   A_stride, B_pool, B_stride, n_adapters, h_in, h_out, r,
                                   scale) -> int:
    """``adapter_ids`` is a HOST address (int32[n], n <= 64); no workspace."""
    return _lib.lib().sgmv_lora_add_host_ids_noalloc(stream, dtype, y, ld_y, x, ld_x,
                                                     adapter_ids, n, A_pool, A_stride, B_pool,
                                                     B_stride, n_adapters, h_in, h_out, r,
                                                     float(scale))


def lora_add_host_ids_noalloc(y, x, ids, A_pool, B_pool, scale: float, stream=None):
    """As ``lora_add_host_ids`` with no workspace: the library's static device scratch
    (calls on one GPU must not overlap in time)."""
    ids_np = np.ascontiguousarray(
        ids.numpy() if hasattr(ids, "numpy") else np.asarray(ids), dtype=np.int32)
    n = int(x.shape[0])
    _check_rows(x, n, "x")
    _check_rows(y, n, "y")
    if ids_np.ndim != 1 or ids_np.shape[0] != n:
        raise ValueError("ids must be a host int32 array [n]")
    r = int(A_pool.shape[1])
    _check_adapters([A_pool[0]], [B_pool[0]], r, int(x.shape[1]), int(y.shape[1]),
                    int(A_pool.shape[0]), int(B_pool.shape[0]))
    st = sgmv_lora_add_host_ids_noalloc(_stream_handle(stream), dtype_code(y), y.data_ptr(),
                                        y.stride(0), x.data_ptr(), x.stride(0), _ptr(ids_np), n,
                                        A_pool.data_ptr(), A_pool.stride(0), B_pool.data_ptr(),
                                        B_pool.stride(0), int(A_pool.shape[0]), x.shape[1],
                                        y.shape[1], r, scale)
    check(st, "sgmv_lora_add_host_ids_noalloc")
    return y
