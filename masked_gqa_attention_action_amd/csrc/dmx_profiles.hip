// Lazily captured graph profiles (OpenDM fast-stack article §5, the default
// backend's row of the comparison table: 16-token buckets, at most 8
// profiles, a profile's first call eager and its second captured).  Host
// code only: a small LRU list of profiles, each holding its graph once
// captured.  The runs go through the public sampler calls.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/dmx.h"

namespace dmx {
int set_last_error(int status, const char* msg);

namespace {
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return set_last_error(status, buf);
}
}  // namespace
}  // namespace dmx

struct dmx_profile_cache {
  struct Entry {
    int64_t key;
    uint64_t fingerprint;
    int calls;        // calls seen since the entry (re)started
    dmx_graph* graph; // after the capturing call
    uint64_t last_use;
  };
  int capacity;
  bool evict;
  uint64_t clock = 0;
  std::vector<Entry> entries;  // unordered; last_use orders them
};

namespace {

constexpr int64_t kNoKey = -1;

uint64_t fnv1a(uint64_t h, uint64_t v) {
  for (int i = 0; i < 8; ++i) {
    h ^= (v >> (8 * i)) & 0xffu;
    h *= 1099511628211ull;
  }
  return h;
}

uint64_t addr(const void* p) { return (uint64_t)(uintptr_t)p; }

// every buffer address a captured run of d binds
uint64_t sampler_fingerprint(const dmx_sampler_desc* d) {
  const dmx_stack_desc* s = d->stack;
  uint64_t h = 1469598103934665603ull;
  for (int l = 0; l < s->n_layers; ++l) {
    const dmx_layer_weights& w = s->layers[l];
    for (const void* p : {(const void*)w.w_mod1, (const void*)w.b_mod1, (const void*)w.w_qkv, (const void*)w.q_norm,
                          (const void*)w.k_norm, (const void*)w.w_o, (const void*)w.w_mod2, (const void*)w.b_mod2,
                          (const void*)w.w_gu, (const void*)w.w_down, (const void*)s->k_pre[l],
                          (const void*)s->v_pre[l]})
      h = fnv1a(h, addr(p));
  }
  for (const void* p : {(const void*)s->mask, (const void*)s->cond, (const void*)s->pos0, (const void*)s->x,
                        (const void*)s->ws, (const void*)s->mod_table, d->sched, (const void*)d->actions,
                        (const void*)d->trajectory})
    h = fnv1a(h, addr(p));
  h = fnv1a(h, (uint64_t)s->ws_bytes);
  h = fnv1a(h, (uint64_t)d->sched_bytes);
  const dmx_sampler_weights* w = d->w;
  h = fnv1a(h, (uint64_t)w->action_dim);
  for (const void* p : {(const void*)w->w_in, (const void*)w->b_in, (const void*)w->w_t1, (const void*)w->b_t1,
                        (const void*)w->w_t2, (const void*)w->b_t2, (const void*)w->w_fmod, (const void*)w->b_fmod,
                        (const void*)w->w_out, (const void*)w->b_out})
    h = fnv1a(h, addr(p));
  return h;
}

int64_t sampler_key(const dmx_sampler_desc* d) {
  const dmx_stack_desc* s = d->stack;
  return (int64_t)s->p_bucket | ((int64_t)s->batch << 16) | ((int64_t)s->chunk << 24) |
         ((int64_t)s->n_steps << 32) | ((int64_t)s->n_layers << 48);
}

void drop_graph(dmx_profile_cache::Entry& e) {
  if (e.graph) dmx_graph_destroy(e.graph);
  e.graph = nullptr;
}

}  // namespace

extern "C" {

int32_t dmx_lazy_bucket(int32_t prefix_len, int32_t max_len) {
  if (prefix_len < 1) return dmx::fail(DMX_ERR_INVALID_ARG, "dmx_lazy_bucket: prefix_len %d < 1", prefix_len);
  if (prefix_len > max_len)
    return dmx::fail(DMX_ERR_PREFIX_TOO_LONG, "dmx_lazy_bucket: prefix_len %d above %d", prefix_len, max_len);
  return (prefix_len + DMX_LAZY_GRANULE - 1) / DMX_LAZY_GRANULE * DMX_LAZY_GRANULE;
}

int dmx_profile_cache_create(int32_t capacity, int32_t evict, dmx_profile_cache** out) {
  if (out == nullptr) return dmx::fail(DMX_ERR_INVALID_ARG, "dmx_profile_cache_create: out is null");
  *out = nullptr;
  if (capacity < 1 || capacity > DMX_LAZY_MAX_PROFILES)
    return dmx::fail(DMX_ERR_INVALID_ARG, "dmx_profile_cache_create: capacity %d not in [1, %d]", capacity,
                     DMX_LAZY_MAX_PROFILES);
  dmx_profile_cache* c = new dmx_profile_cache;
  c->capacity = capacity;
  c->evict = evict != 0;
  c->entries.reserve(DMX_LAZY_MAX_PROFILES);
  *out = c;
  return DMX_OK;
}

void dmx_profile_cache_destroy(dmx_profile_cache* c) {
  if (c == nullptr) return;
  for (auto& e : c->entries) drop_graph(e);
  delete c;
}

int dmx_profile_cache_plan(dmx_profile_cache* c, int64_t key, uint64_t fingerprint, int32_t* action,
                           int64_t* evicted) {
  if (c == nullptr || action == nullptr || evicted == nullptr)
    return dmx::fail(DMX_ERR_INVALID_ARG, "dmx_profile_cache_plan: null argument");
  if (key < 0) return dmx::fail(DMX_ERR_INVALID_ARG, "dmx_profile_cache_plan: key %lld < 0", (long long)key);
  *evicted = kNoKey;
  for (auto& e : c->entries) {
    if (e.key != key) continue;
    e.last_use = ++c->clock;
    if (e.fingerprint != fingerprint) {  // other buffers: the graph is stale
      drop_graph(e);
      e.fingerprint = fingerprint;
      e.calls = 0;
    }
    ++e.calls;
    *action = e.calls == 1 ? DMX_ACTION_EAGER : e.calls == 2 ? DMX_ACTION_CAPTURE : DMX_ACTION_REPLAY;
    return DMX_OK;
  }
  *action = DMX_ACTION_EAGER;
  if ((int)c->entries.size() == c->capacity) {
    if (!c->evict) return DMX_OK;  // runs eager, not kept
    size_t lru = 0;
    for (size_t i = 1; i < c->entries.size(); ++i)
      if (c->entries[i].last_use < c->entries[lru].last_use) lru = i;
    *evicted = c->entries[lru].key;
    drop_graph(c->entries[lru]);
    c->entries.erase(c->entries.begin() + (long)lru);
  }
  c->entries.push_back({key, fingerprint, 1, nullptr, ++c->clock});
  return DMX_OK;
}

int dmx_profile_cache_keys(const dmx_profile_cache* c, int64_t* keys) {
  if (c == nullptr) return dmx::fail(DMX_ERR_INVALID_ARG, "dmx_profile_cache_keys: cache is null");
  if (keys) {
    std::vector<const dmx_profile_cache::Entry*> order;
    for (const auto& e : c->entries) order.push_back(&e);
    for (size_t i = 1; i < order.size(); ++i)  // insertion sort by last use
      for (size_t j = i; j > 0 && order[j]->last_use < order[j - 1]->last_use; --j) std::swap(order[j], order[j - 1]);
    for (size_t i = 0; i < order.size(); ++i) keys[i] = order[i]->key;
  }
  return (int)c->entries.size();
}

int dmx_profile_cache_run_sampler(dmx_profile_cache* c, const dmx_sampler_desc* d, void* stream, int32_t* action) {
  const char* fn = "dmx_profile_cache_run_sampler";
  if (c == nullptr || d == nullptr || d->stack == nullptr || d->w == nullptr || d->stack->layers == nullptr ||
      d->stack->k_pre == nullptr || d->stack->v_pre == nullptr || d->stack->n_layers < 1 ||
      d->stack->n_layers > DMX_MAX_LAYERS)
    return dmx::fail(DMX_ERR_INVALID_ARG, "%s: null or malformed descriptor", fn);
  if (stream == nullptr) return dmx::fail(DMX_ERR_INVALID_ARG, "%s: capture and replay need a non-null stream", fn);
  const int64_t key = sampler_key(d);
  int32_t act = DMX_ACTION_EAGER;
  int64_t evicted = kNoKey;
  int st = dmx_profile_cache_plan(c, key, sampler_fingerprint(d), &act, &evicted);
  if (st != DMX_OK) return st;
  if (action) *action = act;
  dmx_profile_cache::Entry* e = nullptr;
  for (auto& x : c->entries)
    if (x.key == key) e = &x;
  if (act == DMX_ACTION_EAGER) return dmx_sampler_forward(d, stream);
  if (act == DMX_ACTION_CAPTURE) {
    dmx_graph* g = nullptr;
    st = dmx_sampler_graph_create(d, stream, &g);
    if (st != DMX_OK) {
      e->calls = 1;  // the next call tries the capture again
      return st;
    }
    e->graph = g;
  }
  return dmx_graph_launch(e->graph, stream);
}

}  // extern "C"
