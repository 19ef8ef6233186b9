// Expert arena for pools larger than HBM (kimi-k3-in-c README, Part II section 12 "An LRU cache
// for the experts", section 13 "How big should that cache be? Ask the trace"), retargeted from
// NVMe into host memory to an HBM slot arena filled from pinned host memory.
//
// The policy is the pages': a slot holds an expert key, or is EMPTY, or INFLIGHT; a miss takes
// the lowest EMPTY slot, else the least recently used slot that is neither in flight, pinned,
// nor already given to the current batch; a batch reserves serially, fetches its misses in the
// backing store's offset order and publishes each fetched expert in its slot.  Recency is one
// global tick per request.  All of it is host code: an ascending free list, a doubly linked
// list of resident unpinned slots in recency order, and a key -> slot map, so a miss costs
// O(1) instead of a scan over the slots.  The same policy object serves the trace replay, so
// the replayed hit rates are the arena's own.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

#include "k3x_internal.h"

namespace k3x {
namespace {

constexpr int64_t kEmpty = -1;
constexpr int64_t kInflight = -2;

class LruSlots {
 public:
  explicit LruSlots(int n)
      : key_(n, kEmpty), used_(n, 0), pinned_(n, 0), batch_(n, 0), prev_(n, -1), next_(n, -1) {
    free_.reserve(n);
    for (int s = n - 1; s >= 0; --s) free_.push_back(s);  // back() is the lowest slot
  }

  int n() const { return (int)key_.size(); }
  int64_t key(int s) const { return key_[s]; }

  int lookup(int64_t k) const {
    auto it = where_.find(k);
    return it == where_.end() ? -1 : it->second;
  }

  // Starts a batch: its hits and reservations may not be taken by its later misses.
  void begin_batch() { ++batch_id_; }

  // A request for key k: returns its slot and whether it was resident, or -1 when no slot
  // can be given (every slot in flight, pinned or held by this batch).
  int request(int64_t k, bool* hit) {
    int s = lookup(k);
    if (s >= 0) {
      *hit = key_[s] != kInflight;
      if (*hit) touch(s);
      batch_[s] = batch_id_;
      return s;
    }
    *hit = false;
    s = victim();
    if (s < 0) return -1;
    if (key_[s] >= 0) where_.erase(key_[s]);
    key_[s] = kInflight;
    where_[k] = s;
    touch(s);  // recency of a reservation is its request's tick
    batch_[s] = batch_id_;
    return s;
  }

  // Publishes key k in its reserved slot (or frees the slot when the fetch failed).
  void publish(int64_t k, int s, bool ok) {
    if (ok) {
      key_[s] = k;
      if (pin_next_.count(k)) pin(s);
    } else {
      where_.erase(k);
      key_[s] = kEmpty;
      unlink(s);
      free_.push_back(s);
      std::sort(free_.begin(), free_.end(), std::greater<int>());
    }
  }

  // Pinned slots leave the recency list and are never evicted.
  void pin(int s) {
    if (pinned_[s]) return;
    pinned_[s] = 1;
    unlink(s);
  }
  // Keys to pin as soon as they are resident (PIN+LRU).
  void pin_when_resident(int64_t k) { pin_next_[k] = 1; }

 private:
  void unlink(int s) {
    if (prev_[s] < 0 && head_ != s) return;  // not in the list
    if (prev_[s] >= 0) next_[prev_[s]] = next_[s]; else head_ = next_[s];
    if (next_[s] >= 0) prev_[next_[s]] = prev_[s]; else tail_ = prev_[s];
    prev_[s] = next_[s] = -1;
  }
  void touch(int s) {
    used_[s] = ++tick_;
    if (pinned_[s]) return;
    unlink(s);
    prev_[s] = tail_;
    next_[s] = -1;
    if (tail_ >= 0) next_[tail_] = s; else head_ = s;
    tail_ = s;
  }
  int victim() {
    if (!free_.empty()) {
      const int s = free_.back();
      free_.pop_back();
      return s;
    }
    for (int s = head_; s >= 0; s = next_[s])  // oldest first; only this batch's are skipped
      if (key_[s] != kInflight && batch_[s] != batch_id_) return s;
    return -1;
  }

  std::vector<int64_t> key_, used_;
  std::vector<char> pinned_;
  std::vector<int64_t> batch_;
  std::vector<int> prev_, next_, free_;
  std::unordered_map<int64_t, int> where_;
  std::unordered_map<int64_t, char> pin_next_;
  int head_ = -1, tail_ = -1;
  int64_t tick_ = 0, batch_id_ = 0;
};

int64_t belady_hits(const int64_t* trace, int64_t n, int cap) {
  // next_use[i]: index of the next request of trace[i], or n + 1 for never
  std::vector<int64_t> next_use(n);
  std::unordered_map<int64_t, int64_t> last;
  for (int64_t i = n - 1; i >= 0; --i) {
    auto it = last.find(trace[i]);
    next_use[i] = it == last.end() ? n + 1 : it->second;
    last[trace[i]] = i;
  }
  std::unordered_map<int64_t, int64_t> resident;  // key -> its next use
  std::priority_queue<std::pair<int64_t, int64_t>> far;  // (next use, key), stale entries skipped
  int64_t hits = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t k = trace[i];
    auto it = resident.find(k);
    if (it != resident.end()) {
      ++hits;
      it->second = next_use[i];
      far.push({next_use[i], k});
      continue;
    }
    if (cap <= 0) continue;
    if ((int64_t)resident.size() >= cap) {
      while (true) {
        const auto top = far.top();
        far.pop();
        auto r = resident.find(top.second);
        if (r != resident.end() && r->second == top.first) {
          resident.erase(r);
          break;
        }
      }
    }
    resident[k] = next_use[i];
    far.push({next_use[i], k});
  }
  return hits;
}

}  // namespace
}  // namespace k3x

struct k3x_arena {
  k3x::LruSlots* lru = nullptr;
  int32_t n_slots = 0, n_layers = 0, n_experts = 0, max_slots_per_call = 0;
  int64_t slot_bytes = 0, tensor_off[6] = {}, tensor_bytes[6] = {};
  const uint8_t* host[6] = {};
  int64_t host_stride[6] = {};
  bool contiguous = false;  // the six tensors of an expert are back to back in the backing store
  uint8_t* dev = nullptr;   // n_slots * slot_bytes
  k3x_pool* pool = nullptr;
  int32_t* idx_host = nullptr;  // pinned staging [max_slots_per_call]
  int32_t* idx_dev = nullptr;   // remapped ids [max_slots_per_call]
  int64_t hits = 0, misses = 0, bytes = 0;
};

namespace {
thread_local char g_arena_err[256] = "";
}

extern "C" {

size_t k3x_expert_bytes(int32_t hidden, int32_t inter) {
  if (hidden <= 0 || inter <= 0) return 0;
  const int64_t H = hidden, I = inter;
  return (size_t)(2 * (I * H / 2 + I * H / 32) + (H * I / 2 + H * I / 32));
}

k3x_status k3x_arena_create(const k3x_arena_desc* d, k3x_arena** out) {
  if (!d || !out) return K3X_E_INVALID_ARG;
  *out = nullptr;
  if (d->n_slots < 1 || d->n_slots > 8192 || d->n_layers < 1 || d->n_experts < 1 ||
      d->max_slots_per_call < 1 || d->max_slots_per_call > (1 << 26))
    return K3X_E_INVALID_ARG;
  if ((int64_t)d->n_layers * d->n_experts > ((int64_t)1 << 40)) return K3X_E_INVALID_ARG;
  for (int k = 0; k < 6; ++k)
    if (!d->host[k]) return K3X_E_INVALID_ARG;
  const int64_t H = d->hidden, I = d->inter;
  if (H <= 0 || I <= 0 || H % 128 || I % 128 || d->group != 32) return K3X_E_UNSUPPORTED;
  const int64_t tb[6] = {I * H / 2, I * H / 32, I * H / 2, I * H / 32, H * I / 2, H * I / 32};
  k3x_arena* a = new (std::nothrow) k3x_arena;
  if (!a) return K3X_E_INVALID_ARG;
  a->n_slots = d->n_slots;
  a->n_layers = d->n_layers;
  a->n_experts = d->n_experts;
  a->max_slots_per_call = d->max_slots_per_call;
  int64_t off = 0;
  a->contiguous = true;
  for (int k = 0; k < 6; ++k) {
    a->tensor_off[k] = off;
    a->tensor_bytes[k] = tb[k];
    a->host[k] = static_cast<const uint8_t*>(d->host[k]);
    a->host_stride[k] = d->host_stride[k] ? d->host_stride[k] : tb[k];
    if (a->host_stride[k] < tb[k]) {
      delete a;
      return K3X_E_INVALID_ARG;
    }
    if (a->host[k] != a->host[0] + off || a->host_stride[k] != a->host_stride[0])
      a->contiguous = false;
    off += tb[k];
  }
  if (a->contiguous && a->host_stride[0] != off) a->contiguous = false;
  a->slot_bytes = (off + 255) & ~(int64_t)255;
  hipError_t e = hipMalloc(&a->dev, (size_t)a->slot_bytes * a->n_slots);
  if (e == hipSuccess)
    e = hipHostMalloc(reinterpret_cast<void**>(&a->idx_host), sizeof(int32_t) * a->max_slots_per_call);
  if (e == hipSuccess) e = hipMalloc(&a->idx_dev, sizeof(int32_t) * a->max_slots_per_call);
  if (e != hipSuccess) {
    snprintf(g_arena_err, sizeof g_arena_err, "arena_create: %s", hipGetErrorString(e));
    (void)hipFree(a->dev);
    if (a->idx_host) (void)hipHostFree(a->idx_host);
    (void)hipFree(a->idx_dev);
    delete a;
    return K3X_E_HIP;
  }
  k3x_pool_desc pd{};
  pd.n_experts = a->n_slots;  // the pool's experts are the slots
  pd.hidden = d->hidden;
  pd.inter = d->inter;
  pd.group = 32;
  const void** ptrs[6] = {&pd.w1_packed, &pd.w1_scale, &pd.w3_packed, &pd.w3_scale,
                          &pd.w2_packed, &pd.w2_scale};
  for (int k = 0; k < 6; ++k) {
    *ptrs[k] = a->dev + a->tensor_off[k];
    pd.stride_bytes[k] = a->slot_bytes;
  }
  pd.activation = d->activation;
  pd.situ_b1 = d->situ_b1;
  pd.situ_b2 = d->situ_b2;
  k3x_status st = k3x_expert_pool_create(&pd, &a->pool);
  a->lru = new (std::nothrow) k3x::LruSlots(a->n_slots);
  if (st != K3X_OK || !a->lru) {
    k3x_arena_destroy(a);
    return st != K3X_OK ? st : K3X_E_INVALID_ARG;
  }
  *out = a;
  return K3X_OK;
}

void k3x_arena_destroy(k3x_arena* a) {
  if (!a) return;
  if (a->pool) k3x_expert_pool_destroy(a->pool);
  (void)hipFree(a->dev);
  if (a->idx_host) (void)hipHostFree(a->idx_host);
  (void)hipFree(a->idx_dev);
  delete a->lru;
  delete a;
}

const k3x_pool* k3x_arena_pool(const k3x_arena* a) { return a ? a->pool : nullptr; }

k3x_status k3x_arena_getmany(k3x_arena* a, int32_t layer, const int32_t* experts, int32_t n,
                             int32_t* slots_out, int32_t* hits, int32_t* misses, void* stream) {
  if (!a || n < 0 || (n > 0 && (!experts || !slots_out))) return K3X_E_INVALID_ARG;
  if (layer < 0 || layer >= a->n_layers) return K3X_E_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  // phase 1: reserve serially
  std::vector<std::pair<int32_t, int>> fetch;  // (expert, slot)
  int32_t nh = 0, nm = 0;
  a->lru->begin_batch();
  for (int32_t j = 0; j < n; ++j) {
    const int32_t e = experts[j];
    slots_out[j] = -1;
    if (e < 0 || e >= a->n_experts) continue;
    const int64_t k = (int64_t)layer * a->n_experts + e;
    const bool was_reserved = a->lru->lookup(k) >= 0 && a->lru->key(a->lru->lookup(k)) == k3x::kInflight;
    bool hit = false;
    const int slot = a->lru->request(k, &hit);
    slots_out[j] = slot;
    if (slot < 0 || was_reserved) continue;
    if (hit) {
      ++nh;
    } else {
      ++nm;
      fetch.push_back({e, slot});
    }
  }
  // phase 2: fetch in the backing store's offset order (ascending expert within the layer)
  std::sort(fetch.begin(), fetch.end());
  hipError_t err = hipSuccess;
  for (auto& f : fetch) {
    const int64_t ke = (int64_t)layer * a->n_experts + f.first;
    uint8_t* dst = a->dev + (size_t)a->slot_bytes * f.second;
    if (a->contiguous) {  // one coalesced copy of the whole expert
      err = hipMemcpyAsync(dst, a->host[0] + ke * a->host_stride[0], (size_t)a->tensor_off[5] + a->tensor_bytes[5],
                           hipMemcpyHostToDevice, s);
    } else {  // six copies, one per tensor
      for (int k = 0; k < 6 && err == hipSuccess; ++k)
        err = hipMemcpyAsync(dst + a->tensor_off[k], a->host[k] + ke * a->host_stride[k],
                             (size_t)a->tensor_bytes[k], hipMemcpyHostToDevice, s);
    }
    // phase 3: publish what was enqueued (a failed enqueue frees its slot)
    a->lru->publish((int64_t)layer * a->n_experts + f.first, f.second, err == hipSuccess);
    if (err == hipSuccess) a->bytes += a->tensor_off[5] + a->tensor_bytes[5];
  }
  a->hits += nh;
  a->misses += nm;
  if (hits) *hits = nh;
  if (misses) *misses = nm;
  if (err != hipSuccess) {
    snprintf(g_arena_err, sizeof g_arena_err, "arena_getmany: %s", hipGetErrorString(err));
    return K3X_E_HIP;
  }
  return K3X_OK;
}

k3x_status k3x_arena_pin(k3x_arena* a, int32_t layer, int32_t expert) {
  if (!a || layer < 0 || layer >= a->n_layers || expert < 0 || expert >= a->n_experts)
    return K3X_E_INVALID_ARG;
  const int64_t k = (int64_t)layer * a->n_experts + expert;
  const int s = a->lru->lookup(k);
  if (s < 0 || a->lru->key(s) != k) return K3X_E_INVALID_ARG;  // pin resident experts only
  a->lru->pin(s);
  return K3X_OK;
}

k3x_status k3x_arena_stats(const k3x_arena* a, int64_t* hits, int64_t* misses, int64_t* bytes) {
  if (!a) return K3X_E_INVALID_ARG;
  if (hits) *hits = a->hits;
  if (misses) *misses = a->misses;
  if (bytes) *bytes = a->bytes;
  return K3X_OK;
}

k3x_status k3x_arena_moe_forward(k3x_arena* a, int32_t layer, const void* x_bf16, int32_t T,
                                 const int32_t* idx, const float* gates, int32_t topk, float* y,
                                 void* ws, size_t ws_bytes, int32_t* hits, int32_t* misses,
                                 void* stream) {
  if (!a || T < 0 || topk < 1) return K3X_E_INVALID_ARG;
  if ((int64_t)T * topk > a->max_slots_per_call) return K3X_E_UNSUPPORTED;
  if (hits) *hits = 0;
  if (misses) *misses = 0;
  hipStream_t s = (hipStream_t)stream;
  const int32_t n = T * topk;
  if (n > 0) {
    if (!idx) return K3X_E_INVALID_ARG;
    hipError_t e = hipMemcpyAsync(a->idx_host, idx, sizeof(int32_t) * n, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      snprintf(g_arena_err, sizeof g_arena_err, "arena_moe_forward: %s", hipGetErrorString(e));
      return K3X_E_HIP;
    }
    // the batch is the call's distinct experts in slot order (token-major)
    std::vector<int32_t> uniq, slot_of(n, -1);
    std::unordered_map<int32_t, int> pos;
    for (int32_t j = 0; j < n; ++j) {
      const int32_t ex = a->idx_host[j];
      if (ex < 0 || ex >= a->n_experts) continue;
      if (pos.emplace(ex, (int)uniq.size()).second) uniq.push_back(ex);
    }
    std::vector<int32_t> us(uniq.size());
    k3x_status st = k3x_arena_getmany(a, layer, uniq.data(), (int32_t)uniq.size(), us.data(),
                                      hits, misses, stream);
    if (st != K3X_OK) return st;
    for (int32_t j = 0; j < n; ++j) {
      const int32_t ex = a->idx_host[j];
      auto it = (ex >= 0 && ex < a->n_experts) ? pos.find(ex) : pos.end();
      a->idx_host[j] = it == pos.end() ? -1 : us[it->second];  // no slot: the slot is dropped
    }
    e = hipMemcpyAsync(a->idx_dev, a->idx_host, sizeof(int32_t) * n, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) {
      snprintf(g_arena_err, sizeof g_arena_err, "arena_moe_forward: %s", hipGetErrorString(e));
      return K3X_E_HIP;
    }
    // the staging buffer is reused by the next call: wait until this copy has read it
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return K3X_E_HIP;
  }
  return k3x_moe_forward(a->pool, x_bf16, T, a->idx_dev, gates, topk, y, ws, ws_bytes, stream);
}

const char* k3x_arena_last_error(void) { return g_arena_err; }

k3x_status k3x_cache_replay(const int64_t* trace, int64_t n, int32_t cap, int32_t policy,
                            const int64_t* pinned, int32_t n_pinned, int64_t* hits) {
  if (!hits || n < 0 || (n > 0 && !trace) || cap < 0 || (n_pinned > 0 && !pinned))
    return K3X_E_INVALID_ARG;
  if (policy == K3X_CACHE_BELADY) {
    *hits = k3x::belady_hits(trace, n, cap);
    return K3X_OK;
  }
  if (policy != K3X_CACHE_LRU && policy != K3X_CACHE_PIN_LRU) return K3X_E_INVALID_ARG;
  int64_t h = 0;
  if (cap > 0) {
    k3x::LruSlots lru(cap);
    if (policy == K3X_CACHE_PIN_LRU)
      for (int32_t i = 0; i < n_pinned; ++i) lru.pin_when_resident(pinned[i]);
    for (int64_t i = 0; i < n; ++i) {  // one request per batch
      lru.begin_batch();
      bool hit = false;
      const int s = lru.request(trace[i], &hit);
      if (s < 0) continue;
      if (hit) ++h; else lru.publish(trace[i], s, true);
    }
  }
  *hits = h;
  return K3X_OK;
}

k3x_status k3x_cache_replay_batches(const int64_t* keys, const int64_t* batch_start,
                                    int64_t n_batches, int32_t cap, int32_t* slots_out) {
  if (cap < 1 || n_batches < 0 || (n_batches > 0 && (!keys || !batch_start || !slots_out)))
    return K3X_E_INVALID_ARG;
  k3x::LruSlots lru(cap);
  for (int64_t b = 0; b < n_batches; ++b) {
    const int64_t j0 = batch_start[b], j1 = batch_start[b + 1];
    if (j1 < j0) return K3X_E_INVALID_ARG;
    lru.begin_batch();
    std::vector<std::pair<int64_t, int>> fetch;
    for (int64_t j = j0; j < j1; ++j) {
      const int s0 = lru.lookup(keys[j]);
      const bool was_reserved = s0 >= 0 && lru.key(s0) == k3x::kInflight;
      bool hit = false;
      const int s = lru.request(keys[j], &hit);
      slots_out[j] = s;
      if (s >= 0 && !hit && !was_reserved) fetch.push_back({keys[j], s});
    }
    std::sort(fetch.begin(), fetch.end());
    for (auto& f : fetch) lru.publish(f.first, f.second, true);
  }
  return K3X_OK;
}

}  // extern "C"
