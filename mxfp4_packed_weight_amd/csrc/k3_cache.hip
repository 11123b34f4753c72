// Expert cache: packed expert blobs live in host memory, a fixed number of
// HBM slots hold the ones in use. The GPU counterpart of the pages' expert
// cache that streams experts from NVMe into RAM ([ZOR] "How does a
// 2.78-trillion-parameter model fit in 8 GB?", the LRU and its slot
// states; one layer's 896 experts fit in HBM, a whole model's do not).
//
// Policy (CachePolicy, host only, also run alone by k3_cache_replay):
//   - a request names experts; each one is a hit (its slot holds it and the
//     copy has finished), an in-flight reuse (its copy was issued and has
//     not finished: the request waits on that copy instead of issuing a
//     second one) or a miss;
//   - a miss takes an empty slot, else evicts the least recently used slot
//     that is neither pinned nor named by the same request;
//   - every request updates a per-expert histogram and an ordered trace.
// k3_cache_replay_opt runs the same request rules with the optimal offline
// victim (the expert next used farthest ahead, Belady's rule), the bound an
// online policy can be compared against when sizing the cache from a trace
// ([A176] "The interesting design decisions": LRU against Belady over the
// same range of cache sizes).
// Device side (ExpertCache): the slots are one allocation; a miss is an
// asynchronous host-to-device copy on the caller's stream followed by an
// event, and the entries of the device table of expert pointers (what the
// layer kernels read) that changed are written by a one-block kernel on the
// same stream. Entries of experts that are not resident point at an
// all-zero blob, so a kernel handed a stale selection reads zeros rather
// than freed or reused memory. Kernels and copies are ordered by
// that stream, so an evicted slot is overwritten only after the kernels
// queued before the request are done; callers keep one stream per cache.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "k3_internal.h"

namespace k3 {

namespace {

enum class SlotState { kEmpty, kInflight, kReady };

struct SlotInfo {
  int key = -1;
  SlotState st = SlotState::kEmpty;
  uint64_t last_use = 0;
};

// Decisions only: no memory is touched here.
struct CachePolicy {
  enum Kind { kHit, kReuse, kMiss };
  struct Action {
    int expert, slot, evicted;  // evicted: expert that left the slot, or -1
    Kind kind;
  };

  int n_experts = 0;
  std::vector<SlotInfo> slots;
  std::vector<int> slot_of;   // expert -> slot, -1 when not resident
  std::vector<char> pinned;   // per expert
  std::vector<uint64_t> hist;
  std::vector<int32_t> trace;
  uint64_t tick = 0;
  k3_cache_stats st{};

  void init(int n, int n_slots) {
    n_experts = n;
    slots.assign(n_slots, SlotInfo{});
    slot_of.assign(n, -1);
    pinned.assign(n, 0);
    hist.assign(n, 0);
    trace.clear();
    tick = 0;
    st = k3_cache_stats{};
  }

  // Plans a request of `count` experts. `done(slot)` says whether an
  // in-flight copy into that slot has finished. False (nothing changed)
  // when the request cannot be served: more distinct experts than
  // evictable slots.
  template <class Done>
  bool plan(const int32_t *ids, int count, Done done, std::vector<Action> *out) {
    out->clear();
    std::vector<char> named(slots.size(), 0), fresh(slots.size(), 0);
    // slots already holding a named expert stay put during this request
    for (int i = 0; i < count; ++i)
      if (slot_of[ids[i]] >= 0) named[slot_of[ids[i]]] = 1;
    int need = 0;
    {
      std::vector<int> seen;
      for (int i = 0; i < count; ++i)
        if (slot_of[ids[i]] < 0 &&
            std::find(seen.begin(), seen.end(), ids[i]) == seen.end()) {
          seen.push_back(ids[i]);
          ++need;
        }
    }
    int free_slots = 0;
    for (size_t s = 0; s < slots.size(); ++s)
      if (!named[s] && (slots[s].key < 0 || !pinned[slots[s].key])) ++free_slots;
    if (need > free_slots) return false;
    for (int i = 0; i < count; ++i) {
      const int e = ids[i];
      ++st.requests;
      ++hist[e];
      trace.push_back(e);
      int s = slot_of[e];
      if (s >= 0) {
        SlotInfo &si = slots[s];
        // a copy issued by this same request is in flight by definition
        if (si.st == SlotState::kInflight && !fresh[s] && done(s)) si.st = SlotState::kReady;
        const Kind k = si.st == SlotState::kReady ? kHit : kReuse;
        if (k == kHit) ++st.hits;
        else ++st.inflight_reuses;
        si.last_use = ++tick;
        out->push_back(Action{e, s, -1, k});
        continue;
      }
      // miss: an empty slot, else the least recently used evictable one
      s = -1;
      for (size_t j = 0; j < slots.size() && s < 0; ++j)
        if (slots[j].key < 0) s = (int)j;
      if (s < 0) {
        uint64_t best = ~0ull;
        for (size_t j = 0; j < slots.size(); ++j) {
          const SlotInfo &c = slots[j];
          if (named[j] || pinned[c.key]) continue;
          if (c.last_use < best) {
            best = c.last_use;
            s = (int)j;
          }
        }
      }
      SlotInfo &si = slots[s];
      const int ev = si.key;
      if (ev >= 0) {
        slot_of[ev] = -1;
        ++st.evictions;
      }
      si.key = e;
      si.st = SlotState::kInflight;
      si.last_use = ++tick;
      slot_of[e] = s;
      named[s] = 1;
      fresh[s] = 1;
      ++st.misses;
      out->push_back(Action{e, s, ev, kMiss});
    }
    return true;
  }
};

// Table edits of one fetch, passed by value: the launch copies them, so the
// host may plan the next request while this one is still queued.
struct TableEdits {
  static constexpr int kMax = 64;
  int n;
  int expert[kMax];
  const uint8_t *ptr[kMax];
};

__global__ void table_edit_kernel(const uint8_t **table, TableEdits ed) {
  const int i = threadIdx.x;
  if (i < ed.n) table[ed.expert[i]] = ed.ptr[i];
}

}  // namespace

}  // namespace k3

// The handle type of the C interface (declared at global scope there).
struct ExpertCacheImpl {
  std::mutex mu;
  k3::CachePolicy pol;
  size_t bytes = 0;  // per expert blob
  int device = 0;
  uint8_t *slots = nullptr;                // n_slots * bytes, device
  uint8_t *zero = nullptr;                 // one all-zero blob, device
  const uint8_t **table = nullptr;         // n_experts pointers, device
  std::vector<const void *> src;           // host blob per expert
  std::vector<hipEvent_t> ev;              // per slot: its last copy
  std::vector<char> ev_live;
  int32_t *sel_host = nullptr;             // pinned: a batch's selection
  size_t sel_cap = 0;                      // ints sel_host holds
};

namespace k3 {

int32_t *cache_selection_buffer(k3_cache_t c, size_t n) {
  if (!c) return nullptr;
  std::lock_guard<std::mutex> g(c->mu);
  if (n > c->sel_cap) {  // grow (pinned, so the copy into it is a plain DMA)
    if (c->sel_host) (void)hipHostFree(c->sel_host);
    c->sel_host = nullptr;
    c->sel_cap = 0;
    if (hipHostMalloc((void **)&c->sel_host, sizeof(int32_t) * n, hipHostMallocDefault) ==
        hipSuccess)
      c->sel_cap = n;
  }
  return c->sel_host;
}

namespace {

hipError_t flush_edits(const uint8_t **table, TableEdits &ed, hipStream_t stream) {
  if (ed.n == 0) return hipSuccess;
  table_edit_kernel<<<1, TableEdits::kMax, 0, stream>>>(table, ed);
  ed.n = 0;
  return hipGetLastError();
}

hipError_t add_edit(const uint8_t **table, TableEdits &ed, int expert,
                    const uint8_t *ptr, hipStream_t stream) {
  ed.expert[ed.n] = expert;
  ed.ptr[ed.n] = ptr;
  return ++ed.n == TableEdits::kMax ? flush_edits(table, ed, stream) : hipSuccess;
}

}  // namespace

}  // namespace k3

using namespace k3;

extern "C" {

k3_status k3_cache_create(int n_experts, size_t expert_bytes, int n_slots,
                          k3_cache_t *out) {
  const char *fn = "k3_cache_create";
  if (!out) {
    set_error("%s: out is NULL", fn);
    return K3_ERR_ARG;
  }
  *out = nullptr;
  if (n_experts < 1 || n_experts > K3_MAX_EXPERTS || n_slots < 1 ||
      n_slots > n_experts || expert_bytes == 0 || expert_bytes % 256 != 0) {
    set_error("%s: need 1 <= n_slots <= n_experts <= %d and expert_bytes a "
              "positive multiple of 256 (got %d, %d, %zu)",
              fn, K3_MAX_EXPERTS, n_slots, n_experts, expert_bytes);
    return K3_ERR_CONFIG;
  }
  ExpertCacheImpl *c = new (std::nothrow) ExpertCacheImpl;
  if (!c) {
    set_error("%s: host allocation failed", fn);
    return K3_ERR_MEMORY;
  }
  c->pol.init(n_experts, n_slots);
  c->bytes = expert_bytes;
  c->src.assign(n_experts, nullptr);
  c->ev.assign(n_slots, nullptr);
  c->ev_live.assign(n_slots, 0);
  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess) e = hipMalloc((void **)&c->slots, (size_t)n_slots * expert_bytes);
  if (e == hipSuccess) e = hipMalloc((void **)&c->table, sizeof(void *) * n_experts);
  // entries of experts that are not resident point at an all-zero blob
  // (it decodes to zero weights), never at NULL or at a reused slot
  if (e == hipSuccess) e = hipMalloc((void **)&c->zero, expert_bytes);
  if (e == hipSuccess) e = hipMemset(c->zero, 0, expert_bytes);
  if (e == hipSuccess) {
    std::vector<const uint8_t *> init(n_experts, c->zero);
    e = hipMemcpy(c->table, init.data(), sizeof(void *) * n_experts,
                  hipMemcpyHostToDevice);
  }
  for (int s = 0; e == hipSuccess && s < n_slots; ++s)
    e = hipEventCreateWithFlags(&c->ev[s], hipEventDisableTiming);
  if (e == hipSuccess)
    e = hipHostMalloc((void **)&c->sel_host, sizeof(int32_t) * K3_MAX_TOPK,
                      hipHostMallocDefault);
  if (e == hipSuccess) c->sel_cap = K3_MAX_TOPK;
  if (e != hipSuccess) {
    k3_cache_destroy(c);
    return device_status(e, fn);
  }
  *out = c;
  return K3_OK;
}

void k3_cache_destroy(k3_cache_t c) {
  if (!c) return;
  for (hipEvent_t ev : c->ev)
    if (ev) (void)hipEventDestroy(ev);
  if (c->slots) (void)hipFree(c->slots);
  if (c->zero) (void)hipFree(c->zero);
  if (c->table) (void)hipFree((void *)c->table);
  if (c->sel_host) (void)hipHostFree(c->sel_host);
  delete c;
}

k3_status k3_cache_set_source(k3_cache_t c, int expert, const void *host_blob) {
  if (!c || expert < 0 || expert >= c->pol.n_experts || !host_blob) {
    set_error("k3_cache_set_source: bad cache, expert index or NULL blob");
    return K3_ERR_ARG;
  }
  std::lock_guard<std::mutex> g(c->mu);
  c->src[expert] = host_blob;
  return K3_OK;
}

k3_status k3_cache_pin(k3_cache_t c, int expert, int pinned) {
  if (!c || expert < 0 || expert >= c->pol.n_experts) {
    set_error("k3_cache_pin: bad cache or expert index");
    return K3_ERR_ARG;
  }
  std::lock_guard<std::mutex> g(c->mu);
  c->pol.pinned[expert] = pinned ? 1 : 0;
  return K3_OK;
}

k3_status k3_cache_fetch(k3_cache_t c, const int32_t *ids, int count,
                         k3_stream_t stream) {
  const char *fn = "k3_cache_fetch";
  if (!c || !ids || count < 1) {
    set_error("%s: bad cache, NULL ids or count < 1", fn);
    return K3_ERR_ARG;
  }
  std::lock_guard<std::mutex> g(c->mu);
  for (int i = 0; i < count; ++i) {
    if (ids[i] < 0 || ids[i] >= c->pol.n_experts) {
      set_error("%s: expert %d outside [0, %d)", fn, ids[i], c->pol.n_experts);
      return K3_ERR_ARG;
    }
    if (!c->src[ids[i]] && c->pol.slot_of[ids[i]] < 0) {
      set_error("%s: expert %d has no host source", fn, ids[i]);
      return K3_ERR_CONFIG;
    }
  }
  std::vector<CachePolicy::Action> acts;
  auto done = [&](int s) {
    return !c->ev_live[s] || hipEventQuery(c->ev[s]) == hipSuccess;
  };
  if (!c->pol.plan(ids, count, done, &acts))
    return (set_error("%s: %d slots cannot hold this request beside the pinned "
                      "experts (a cache with more slots would serve it)",
                      fn, (int)c->pol.slots.size()),
            K3_ERR_MEMORY);
  hipError_t e = hipSuccess;
  TableEdits ed;
  ed.n = 0;
  for (const CachePolicy::Action &a : acts) {
    if (a.kind == CachePolicy::kReuse) {
      // the copy is on its way: this stream waits for it, no second copy
      if (c->ev_live[a.slot]) e = hipStreamWaitEvent(stream, c->ev[a.slot], 0);
    } else if (a.kind == CachePolicy::kMiss) {
      if (c->ev_live[a.slot]) e = hipStreamWaitEvent(stream, c->ev[a.slot], 0);
      if (e == hipSuccess && a.evicted >= 0)
        e = add_edit(c->table, ed, a.evicted, c->zero, stream);
      uint8_t *dst = c->slots + (size_t)a.slot * c->bytes;
      if (e == hipSuccess)
        e = hipMemcpyAsync(dst, c->src[a.expert], c->bytes, hipMemcpyHostToDevice,
                           stream);
      if (e == hipSuccess) e = hipEventRecord(c->ev[a.slot], stream);
      if (e == hipSuccess) e = add_edit(c->table, ed, a.expert, dst, stream);
      c->ev_live[a.slot] = 1;
      c->pol.st.bytes_copied += c->bytes;
    }
    if (e != hipSuccess) return device_status(e, fn);
  }
  return device_status(flush_edits(c->table, ed, stream), fn);
}

const uint8_t *const *k3_cache_table(k3_cache_t c) { return c ? c->table : nullptr; }

k3_status k3_cache_get_stats(k3_cache_t c, k3_cache_stats *out) {
  if (!c || !out) return (set_error("k3_cache_get_stats: NULL argument"), K3_ERR_ARG);
  std::lock_guard<std::mutex> g(c->mu);
  *out = c->pol.st;
  return K3_OK;
}

k3_status k3_cache_histogram(k3_cache_t c, uint64_t *counts) {
  if (!c || !counts) return (set_error("k3_cache_histogram: NULL argument"), K3_ERR_ARG);
  std::lock_guard<std::mutex> g(c->mu);
  memcpy(counts, c->pol.hist.data(), sizeof(uint64_t) * c->pol.n_experts);
  return K3_OK;
}

k3_status k3_cache_trace(k3_cache_t c, int32_t *buf, size_t cap, size_t *len) {
  if (!c || !len) return (set_error("k3_cache_trace: NULL argument"), K3_ERR_ARG);
  std::lock_guard<std::mutex> g(c->mu);
  *len = c->pol.trace.size();
  if (buf) memcpy(buf, c->pol.trace.data(), sizeof(int32_t) * std::min(cap, *len));
  return K3_OK;
}

k3_status k3_cache_replay(const int32_t *trace, size_t len, int n_experts,
                          int n_slots, const int32_t *pinned, int n_pinned,
                          int request_size, k3_cache_stats *out) {
  const char *fn = "k3_cache_replay";
  if (!trace || !out || (n_pinned > 0 && !pinned))
    return (set_error("%s: NULL argument", fn), K3_ERR_ARG);
  if (n_experts < 1 || n_slots < 1 || n_slots > n_experts || request_size < 1)
    return (set_error("%s: need 1 <= n_slots <= n_experts and request_size >= 1", fn),
            K3_ERR_CONFIG);
  CachePolicy p;
  p.init(n_experts, n_slots);
  for (int i = 0; i < n_pinned; ++i) {
    if (pinned[i] < 0 || pinned[i] >= n_experts)
      return (set_error("%s: pinned expert %d outside [0, %d)", fn, pinned[i], n_experts),
              K3_ERR_ARG);
    p.pinned[pinned[i]] = 1;
  }
  std::vector<CachePolicy::Action> acts;
  for (size_t i = 0; i < len; i += request_size) {
    const int cnt = (int)std::min<size_t>(request_size, len - i);
    for (int j = 0; j < cnt; ++j)
      if (trace[i + j] < 0 || trace[i + j] >= n_experts)
        return (set_error("%s: trace entry %zu = %d outside [0, %d)", fn, i + j,
                          trace[i + j], n_experts),
                K3_ERR_ARG);
    // a replay has no copies in flight: every copy has finished
    if (!p.plan(trace + i, cnt, [](int) { return true; }, &acts))
      return (set_error("%s: request at %zu does not fit %d slots", fn, i, n_slots),
              K3_ERR_MEMORY);
  }
  *out = p.st;
  return K3_OK;
}

k3_status k3_cache_replay_opt(const int32_t *trace, size_t len, int n_experts,
                              int n_slots, const int32_t *pinned, int n_pinned,
                              int request_size, k3_cache_stats *out) {
  const char *fn = "k3_cache_replay_opt";
  if (!trace || !out || (n_pinned > 0 && !pinned))
    return (set_error("%s: NULL argument", fn), K3_ERR_ARG);
  if (n_experts < 1 || n_slots < 1 || n_slots > n_experts || request_size < 1)
    return (set_error("%s: need 1 <= n_slots <= n_experts and request_size >= 1", fn),
            K3_ERR_CONFIG);
  for (size_t i = 0; i < len; ++i)
    if (trace[i] < 0 || trace[i] >= n_experts)
      return (set_error("%s: trace entry %zu = %d outside [0, %d)", fn, i, trace[i], n_experts),
              K3_ERR_ARG);
  std::vector<char> pin(n_experts, 0);
  for (int i = 0; i < n_pinned; ++i) {
    if (pinned[i] < 0 || pinned[i] >= n_experts)
      return (set_error("%s: pinned expert %d outside [0, %d)", fn, pinned[i], n_experts),
              K3_ERR_ARG);
    pin[pinned[i]] = 1;
  }
  // next_pos[i]: the next position of trace[i] after i (len when none)
  std::vector<size_t> next_pos(len), last(n_experts, len);
  for (size_t i = len; i-- > 0;) {
    next_pos[i] = last[trace[i]];
    last[trace[i]] = i;
  }
  // next use of each expert from the current position on
  std::vector<size_t> next_use(last);
  std::vector<int> holder(n_slots, -1), slot_of(n_experts, -1);
  k3_cache_stats st{};
  for (size_t r0 = 0; r0 < len; r0 += request_size) {
    const size_t r1 = std::min(len, r0 + (size_t)request_size);
    // whole request: every named expert must be resident at once
    std::vector<char> named(n_slots, 0), fresh(n_slots, 0);
    int need = 0;
    for (size_t i = r0; i < r1; ++i) {
      const int e = trace[i];
      if (slot_of[e] >= 0) named[slot_of[e]] = 1;
    }
    {
      std::vector<int> seen;
      for (size_t i = r0; i < r1; ++i)
        if (slot_of[trace[i]] < 0 &&
            std::find(seen.begin(), seen.end(), trace[i]) == seen.end()) {
          seen.push_back(trace[i]);
          ++need;
        }
    }
    int free_slots = 0;
    for (int j = 0; j < n_slots; ++j)
      if (!named[j] && (holder[j] < 0 || !pin[holder[j]])) ++free_slots;
    if (need > free_slots)
      return (set_error("%s: request at %zu does not fit %d slots", fn, r0, n_slots),
              K3_ERR_MEMORY);
    for (size_t i = r0; i < r1; ++i) {
      const int e = trace[i];
      ++st.requests;
      next_use[e] = next_pos[i];
      int s = slot_of[e];
      if (s >= 0) {
        if (fresh[s]) ++st.inflight_reuses;
        else ++st.hits;
        continue;
      }
      // an empty slot, else the evictable slot whose expert is next used
      // farthest ahead (never again counts as farthest); ties: lowest slot
      for (int j = 0; j < n_slots && s < 0; ++j)
        if (holder[j] < 0) s = j;
      if (s < 0) {
        size_t best = 0;
        for (int j = 0; j < n_slots; ++j) {
          if (named[j] || pin[holder[j]]) continue;
          const size_t nu = next_use[holder[j]];
          if (s < 0 || nu > best) {
            best = nu;
            s = j;
          }
        }
        slot_of[holder[s]] = -1;
        ++st.evictions;
      }
      holder[s] = e;
      slot_of[e] = s;
      named[s] = fresh[s] = 1;
      ++st.misses;
    }
  }
  *out = st;
  return K3_OK;
}

}  // extern "C"
