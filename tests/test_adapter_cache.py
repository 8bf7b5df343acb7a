"""The native adapter slot cache (sgmv_slot_cache_*: host bookkeeping of which adapter key
occupies which slot of a device pool), against a plain model of its documented policy:
a key that is not resident takes the lowest free slot, else the least recently used slot
whose key the batch does not use (ties: the lowest slot)."""
import numpy as np
import pytest

from adapter_gemv_amd import _lib
from adapter_gemv_amd.adapter_pool import SlotCache


class Model:
    """The policy written out with Python lists (the slot of each key, the batch number of
    each slot's last use)."""

    def __init__(self, n):
        self.key = [None] * n
        self.last = [0] * n
        self.clock = 0

    def map(self, keys):
        self.clock += 1
        distinct = list(dict.fromkeys(keys))
        if len(distinct) > len(self.key):
            return None
        resident = {k: s for s, k in enumerate(self.key) if k is not None}
        busy = {resident[k] for k in distinct if k in resident}
        misses = []
        for k in distinct:
            if k in resident:
                continue
            free = [s for s, kk in enumerate(self.key) if kk is None]
            if free:
                s = free[0]
            else:
                cand = [s for s in range(len(self.key)) if s not in busy]
                s = min(cand, key=lambda q: (self.last[q], q))
                del resident[self.key[s]]
            self.key[s] = k
            resident[k] = s
            busy.add(s)
            misses.append((k, s))
        for k in distinct:
            self.last[resident[k]] = self.clock
        return [resident[k] for k in keys], misses


def test_hand_sequence():
    c = SlotCache(4)
    slots, mk, ms = c.map([10, 20, 30, 20])
    assert slots.tolist() == [0, 1, 2, 1] and mk.tolist() == [10, 20, 30] and ms.tolist() == [0, 1, 2]
    slots, mk, ms = c.map([20, 40])                     # 40 takes the free slot 3
    assert slots.tolist() == [1, 3] and mk.tolist() == [40]
    slots, mk, ms = c.map([50])                         # LRU: 10 and 30 (batch 1), lowest slot
    assert slots.tolist() == [0] and mk.tolist() == [50] and c.lookup(10) == -1
    slots, mk, ms = c.map([10, 30, 50, 40])             # 10 cannot take a slot the batch uses
    assert slots.tolist() == [1, 2, 0, 3] and mk.tolist() == [10] and c.lookup(20) == -1
    with pytest.raises(_lib.SgmvError) as e:            # five distinct keys, four slots
        c.map([1, 2, 3, 4, 5])
    assert e.value.status == _lib.ERR_SHAPE
    assert [c.lookup(k) for k in (10, 30, 50, 40)] == [1, 2, 0, 3]   # nothing changed
    c.evict(30)
    assert c.lookup(30) == -1
    slots, mk, ms = c.map([60])                         # the freed slot
    assert slots.tolist() == [2] and mk.tolist() == [60]
    with pytest.raises(_lib.SgmvError):
        c.evict(12345)
    slots, mk, ms = c.map([])
    assert slots.size == 0 and mk.size == 0
    c.close()


@pytest.mark.parametrize("n_slots,universe,seed", [(1, 3, 0), (5, 9, 1), (16, 40, 2), (64, 70, 3)])
def test_random_batches_follow_the_policy(n_slots, universe, seed):
    rng = np.random.default_rng(seed)
    c, m = SlotCache(n_slots), Model(n_slots)
    for _ in range(300):
        n = int(rng.integers(0, 2 * n_slots + 2))
        keys = [int(k) * 7919 - 3 for k in rng.integers(0, universe, n)]
        want = m.map(keys)
        if want is None:
            with pytest.raises(_lib.SgmvError):
                c.map(keys)
            continue
        slots, mk, ms = c.map(keys)
        assert slots.tolist() == want[0]
        assert list(zip(mk.tolist(), ms.tolist())) == want[1]
    c.close()


def test_rejects():
    L = _lib.lib()
    assert L.sgmv_slot_cache_create(0, None) == _lib.ERR_NULL
    import ctypes
    h = ctypes.c_void_p()
    assert L.sgmv_slot_cache_create(0, ctypes.byref(h)) == _lib.ERR_SHAPE and not h.value
    assert L.sgmv_slot_cache_map(None, None, 0, None, None, None, None) == _lib.ERR_NULL


def test_upload_rejects_before_any_hip_call():
    L = _lib.lib()
    P, H = 1 << 40, 2 << 40
    ok = dict(stream=None, A_pool=P, A_stride=16 * 4096, B_pool=P + (1 << 30), B_stride=16 * 4096,
              slot=3, n_slots=8, A_host=H, B_host=H + (1 << 20), r=16, h_in=4096, h_out=4096)

    def up(**kw):
        a = dict(ok)
        a.update(kw)
        return L.sgmv_upload_adapter(*a.values())

    assert up(slot=8) == _lib.ERR_SHAPE
    assert up(slot=-1) == _lib.ERR_SHAPE
    assert up(r=8) == _lib.ERR_UNSUPPORTED
    assert up(A_stride=16 * 4096 - 8) == _lib.ERR_SHAPE
    assert up(B_stride=16 * 4096 + 4) == _lib.ERR_ALIGNMENT
    assert up(A_host=None) == _lib.ERR_NULL
    assert up(B_pool=P + 8) == _lib.ERR_ALIGNMENT
    assert up(h_in=4092) == _lib.ERR_ALIGNMENT
