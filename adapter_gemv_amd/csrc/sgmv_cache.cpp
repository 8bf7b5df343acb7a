// Adapter slot cache (host only): which adapter occupies which slot of a device adapter
// pool.  The Punica paper summary (research.elamur.ai, "Summary" and "Key points") has the
// runner fetch only the small LoRA matrices of an adapter, on demand, when a request needs
// it; this is the bookkeeping of that step on one GPU.  A batch's adapter keys are mapped
// to pool slots; a key that is not resident takes a free slot or, failing that, the least
// recently used slot whose adapter the batch does not use, and is reported back so that the
// caller uploads it (sgmv_upload_adapter) before the SGMV call on the same stream.
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/sgmv.h"

struct sgmv_slot_cache {
  std::unordered_map<int64_t, int32_t> slot_of;  // resident key -> slot
  std::vector<int64_t> key;                      // per slot: its key (valid if used)
  std::vector<char> used;                        // per slot: holds an adapter
  std::vector<uint64_t> last;                    // per slot: stamp of its last batch
  std::vector<uint64_t> mark;                    // per slot: stamp of the batch that uses it
  uint64_t clock = 0;
};

extern "C" int sgmv_slot_cache_create(int32_t n_slots, sgmv_slot_cache** cache) {
  if (!cache) return SGMV_ERR_NULL;
  *cache = nullptr;
  if (n_slots <= 0 || n_slots > (1 << 24)) return SGMV_ERR_SHAPE;
  sgmv_slot_cache* c = new (std::nothrow) sgmv_slot_cache;
  if (!c) return SGMV_ERR_SHAPE;
  const size_t n = static_cast<size_t>(n_slots);
  c->key.assign(n, 0);
  c->used.assign(n, 0);
  c->last.assign(n, 0);
  c->mark.assign(n, 0);
  *cache = c;
  return SGMV_OK;
}

extern "C" void sgmv_slot_cache_destroy(sgmv_slot_cache* cache) { delete cache; }

extern "C" int sgmv_slot_cache_lookup(const sgmv_slot_cache* cache, int64_t key, int32_t* slot) {
  if (!cache || !slot) return SGMV_ERR_NULL;
  const auto it = cache->slot_of.find(key);
  *slot = it == cache->slot_of.end() ? -1 : it->second;
  return SGMV_OK;
}

extern "C" int sgmv_slot_cache_evict(sgmv_slot_cache* cache, int64_t key) {
  if (!cache) return SGMV_ERR_NULL;
  const auto it = cache->slot_of.find(key);
  if (it == cache->slot_of.end()) return SGMV_ERR_ADAPTER_ID;
  cache->used[it->second] = 0;
  cache->slot_of.erase(it);
  return SGMV_OK;
}

extern "C" int sgmv_slot_cache_map(sgmv_slot_cache* cache, const int64_t* keys, int32_t n,
                                   int32_t* slots, int64_t* miss_keys, int32_t* miss_slots,
                                   int32_t* n_miss) {
  if (!cache || !n_miss) return SGMV_ERR_NULL;
  if (n < 0) return SGMV_ERR_SHAPE;
  if (n > 0 && (!keys || !slots || !miss_keys || !miss_slots)) return SGMV_ERR_NULL;
  sgmv_slot_cache& c = *cache;
  const int32_t n_slots = static_cast<int32_t>(c.key.size());
  const uint64_t stamp = ++c.clock;
  // the batch's distinct keys: resident ones are marked as used by this batch; count the
  // others (each needs a slot no key of the batch holds)
  std::unordered_map<int64_t, int32_t> fresh;  // non-resident key -> its slot, once chosen
  int32_t distinct = 0;
  for (int32_t t = 0; t < n; ++t) {
    const auto it = c.slot_of.find(keys[t]);
    if (it != c.slot_of.end()) {
      if (c.mark[it->second] != stamp) ++distinct;
      c.mark[it->second] = stamp;
    } else if (fresh.emplace(keys[t], -1).second) {
      ++distinct;
    }
  }
  if (distinct > n_slots) return SGMV_ERR_SHAPE;  // no slot or key changed
  // slots for the non-resident keys, in the order they first appear in the batch: a free
  // slot (lowest index) if any, else the least recently used slot the batch does not use
  int32_t misses = 0;
  for (int32_t t = 0; t < n; ++t) {
    auto it = fresh.find(keys[t]);
    if (it == fresh.end() || it->second >= 0) continue;
    int32_t pick = -1;
    for (int32_t s = 0; s < n_slots; ++s)
      if (!c.used[s]) {
        pick = s;
        break;
      }
    if (pick < 0) {
      for (int32_t s = 0; s < n_slots; ++s)
        if (c.mark[s] != stamp && (pick < 0 || c.last[s] < c.last[pick])) pick = s;
      c.slot_of.erase(c.key[pick]);  // the evicted adapter
    }
    c.used[pick] = 1;
    c.key[pick] = keys[t];
    c.mark[pick] = stamp;
    c.slot_of[keys[t]] = pick;
    it->second = pick;
    miss_keys[misses] = keys[t];
    miss_slots[misses] = pick;
    ++misses;
  }
  for (int32_t t = 0; t < n; ++t) {
    const int32_t s = c.slot_of.find(keys[t])->second;
    slots[t] = s;
    c.last[s] = stamp;
  }
  *n_miss = misses;
  return SGMV_OK;
}
