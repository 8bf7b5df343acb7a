"""On-demand adapter loading into a device adapter pool (argument marshalling over
libsgmv's slot cache and upload calls; see include/sgmv.h).

The Punica paper summary (research.elamur.ai, "Summary" and "Key points") has the runner
fetch only the small LoRA matrices of an adapter when a request needs it, which takes
milliseconds.  ``AdapterPool`` is that step on one GPU for one projection:

* adapters are registered from host memory, kept in pinned host buffers (torch
  ``pin_memory``), under any integer key;
* the device pool holds ``n_slots`` adapters, stacked over ``layers`` layers:
  A ``[layers, n_slots, r, h_in]`` and B ``[layers, n_slots, h_out, r]`` (layer l's pools
  are ``A[l]`` / ``B[l]``, the pointer offset the header describes for stacked pools);
* ``prepare(keys)`` maps a batch's keys to slots with the native LRU slot cache and
  enqueues the uploads of the adapters that were not resident, on the caller's stream;
* ``lora_add(y, x, slots, scale, layer)`` then runs SGMV on those slots (one launch with
  host ids for up to 64 tokens, device ids above).
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from . import _lib, sgmv
from ._lib import check


class SlotCache:
    """ctypes handle of a native sgmv_slot_cache (host LRU map of adapter keys to slots)."""

    def __init__(self, n_slots: int):
        h = ctypes.c_void_p()
        check(_lib.lib().sgmv_slot_cache_create(int(n_slots), ctypes.byref(h)),
              "sgmv_slot_cache_create")
        self._h = h
        self.n_slots = int(n_slots)

    def close(self) -> None:
        if self._h:
            _lib.lib().sgmv_slot_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def map(self, keys) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(slots int32[n], miss_keys int64[m], miss_slots int32[m]) for a batch's keys."""
        k = np.ascontiguousarray(np.asarray(keys), dtype=np.int64)
        n = int(k.shape[0])
        slots = np.zeros(max(n, 1), np.int32)
        mk = np.zeros(max(n, 1), np.int64)
        ms = np.zeros(max(n, 1), np.int32)
        m = np.zeros(1, np.int32)
        check(_lib.lib().sgmv_slot_cache_map(self._h, k.ctypes.data, n, slots.ctypes.data,
                                             mk.ctypes.data, ms.ctypes.data, m.ctypes.data),
              "sgmv_slot_cache_map")
        c = int(m[0])
        return slots[:n].copy(), mk[:c].copy(), ms[:c].copy()

    def lookup(self, key: int) -> int:
        s = np.zeros(1, np.int32)
        check(_lib.lib().sgmv_slot_cache_lookup(self._h, int(key), s.ctypes.data),
              "sgmv_slot_cache_lookup")
        return int(s[0])

    def evict(self, key: int) -> None:
        check(_lib.lib().sgmv_slot_cache_evict(self._h, int(key)), "sgmv_slot_cache_evict")


class AdapterPool:
    """A device pool of ``n_slots`` LoRA adapters (rank r, h_in -> h_out) over ``layers``
    layers, filled on demand from registered host copies."""

    def __init__(self, n_slots: int, r: int, h_in: int, h_out: int, layers: int = 1,
                 dtype=None, device="cuda"):
        import torch
        dtype = torch.bfloat16 if dtype is None else dtype
        self.r, self.h_in, self.h_out, self.layers = int(r), int(h_in), int(h_out), int(layers)
        self.device = torch.device(device)
        self.A = torch.zeros((layers, n_slots, r, h_in), dtype=dtype, device=self.device)
        self.B = torch.zeros((layers, n_slots, h_out, r), dtype=dtype, device=self.device)
        self.cache = SlotCache(n_slots)
        self._host: Dict[int, Tuple[object, object]] = {}
        self.stats = {"hits": 0, "misses": 0, "uploaded_bytes": 0}

    @property
    def n_slots(self) -> int:
        return self.cache.n_slots

    def register(self, key: int, A, B) -> None:
        """Keep a pinned host copy of adapter ``key``: A ``[layers, r, h_in]`` (or ``[r,
        h_in]`` for one layer) and B ``[layers, h_out, r]``, CPU tensors of the pool's
        dtype.  A registered key's device copy is refreshed on its next miss."""
        import torch
        A = A.reshape(self.layers, self.r, self.h_in)
        B = B.reshape(self.layers, self.h_out, self.r)
        if A.dtype != self.A.dtype or B.dtype != self.B.dtype:
            raise TypeError("adapter dtype differs from the pool's")
        a = torch.empty(A.shape, dtype=A.dtype, pin_memory=True)
        b = torch.empty(B.shape, dtype=B.dtype, pin_memory=True)
        a.copy_(A)
        b.copy_(B)
        self._host[int(key)] = (a, b)
        if self.cache.lookup(key) >= 0:
            self.cache.evict(key)      # the device copy is stale

    def prepare(self, keys: Sequence[int], stream=None) -> np.ndarray:
        """Slots of a batch's adapter keys (int32 [n]); adapters that were not resident are
        uploaded from their pinned host copies on ``stream`` (default: the current one),
        ahead of any SGMV call enqueued after this on that stream."""
        keys = np.asarray(keys, dtype=np.int64)
        for k in np.unique(keys):
            if int(k) not in self._host:
                raise KeyError(f"adapter {int(k)} is not registered")
        slots, miss_keys, miss_slots = self.cache.map(keys)
        st = sgmv._stream_handle(stream)
        L = _lib.lib()
        a_st, b_st = self.A.stride(1), self.B.stride(1)
        esz = self.A.element_size()
        for key, slot in zip(miss_keys.tolist(), miss_slots.tolist()):
            a, b = self._host[key]
            for layer in range(self.layers):
                rc = L.sgmv_upload_adapter(st, self.A[layer].data_ptr(), a_st, self.B[layer].data_ptr(),
                                           b_st, slot, self.n_slots, a[layer].data_ptr(),
                                           b[layer].data_ptr(), self.r, self.h_in, self.h_out)
                check(rc, "sgmv_upload_adapter")
            self.stats["uploaded_bytes"] += esz * (a.numel() + b.numel())
        distinct = int(np.unique(keys).size)
        self.stats["misses"] += int(miss_keys.size)
        self.stats["hits"] += distinct - int(miss_keys.size)
        return slots

    def layer_pools(self, layer: int = 0):
        """Layer ``layer``'s pools: views ``[n_slots, r, h_in]`` and ``[n_slots, h_out, r]``."""
        return self.A[layer], self.B[layer]

    def lora_add(self, y, x, slots: np.ndarray, scale: float, layer: int = 0,
                 workspace=None, stream=None):
        """y[t] += scale * (x[t] @ A[slots[t]]) @ B[slots[t]] with layer ``layer``'s
        adapters: one launch with the slots in its arguments for up to 64 tokens, device
        slot ids (device grouping + table kernels) above."""
        import torch
        A, B = self.layer_pools(layer)
        n = int(x.shape[0])
        if n <= sgmv.DECODE_MAX_TOKENS:
            return sgmv.lora_add_host_ids(y, x, np.asarray(slots, np.int32), A, B, scale,
                                          workspace, stream)
        ids = torch.as_tensor(np.asarray(slots, np.int32), device=x.device)
        return sgmv.lora_add_pool(y, x, ids, A, B, scale, workspace, stream)

    def close(self) -> None:
        self.cache.close()
