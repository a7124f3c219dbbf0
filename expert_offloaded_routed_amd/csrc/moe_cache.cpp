// Slot-cache policy (host only): LRU / LFRU victims, bounded refills per step, fixed-lag
// visibility.  The rules are spelled out in include/moe.h (moe_cache_policy_step).
#include <hip/hip_runtime_api.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
moe_status fail(moe_status st, const char* fmt, ...);
moe_status ok();
moe_status check_shape(const moe_shape* s);
}  // namespace moe

using namespace moe;

struct moe_cache {
  int E, S, K;
  moe_cache_config cfg;
  std::vector<int32_t> slot_expert;  // [S], -1 empty or being refilled
  std::vector<int32_t> expert_slot;  // [E], -1 cold
  std::vector<int64_t> last_use;     // [S], -1 never
  std::vector<int64_t> freq;         // [E] (LFRU)
  struct Pending {
    int32_t expert, slot;
    int64_t visible;
  };
  std::vector<Pending> pending;  // in planning order
  moe_cache_stats stats;
  int64_t last_step;
  bool stepped;
  // scratch
  std::vector<int32_t> count;    // [E] routes of the observed step
  std::vector<int32_t> touched;  // experts routed at this step
  std::vector<uint8_t> used;     // [S]
};

static bool slot_pending(const moe_cache* c, int s) {
  for (const auto& p : c->pending)
    if (p.slot == s) return true;
  return false;
}

static bool expert_pending(const moe_cache* c, int e) {
  for (const auto& p : c->pending)
    if (p.expert == e) return true;
  return false;
}

static int choose_victim(const moe_cache* c) {
  for (int s = 0; s < c->S; ++s)
    if (c->slot_expert[s] < 0 && !slot_pending(c, s)) return s;
  int best = -1;
  int64_t bf = 0, bl = 0;
  for (int s = 0; s < c->S; ++s) {
    if (c->slot_expert[s] < 0 || c->used[s] || slot_pending(c, s)) continue;
    const int64_t f = c->cfg.policy == MOE_POLICY_LFRU ? c->freq[c->slot_expert[s]] : 0;
    const int64_t l = c->last_use[s];
    // keys compare as (freq, last_use, slot); slot order is the scan order
    if (best < 0 || f < bf || (f == bf && l < bl)) {
      best = s;
      bf = f;
      bl = l;
    }
  }
  return best;
}

extern "C" {

moe_status moe_cache_create(const moe_shape* shape, const moe_cache_config* config,
                            const int32_t* initial_slot_expert, moe_cache** out) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!config || !out) return fail(MOE_ERR_INVALID_ARG, "moe_cache_create: NULL config or out");
  if (config->policy != MOE_POLICY_LRU && config->policy != MOE_POLICY_LFRU)
    return fail(MOE_ERR_INVALID_ARG, "unknown policy %d", config->policy);
  if (config->max_refills_per_step < 0 || config->lag_steps < 1 || config->max_pending < 1 ||
      config->decay_period < 0)
    return fail(MOE_ERR_INVALID_ARG, "cache config out of range (R=%d L=%d Q=%d decay=%d)",
                config->max_refills_per_step, config->lag_steps, config->max_pending,
                config->decay_period);
  moe_cache* c = new moe_cache();
  c->E = shape->n_experts;
  c->S = shape->n_slots;
  c->K = shape->top_k;
  c->cfg = *config;
  c->slot_expert.assign(c->S, -1);
  c->expert_slot.assign(c->E, -1);
  c->last_use.assign(c->S, -1);
  c->freq.assign(c->E, 0);
  c->count.assign(c->E, 0);
  c->used.assign(c->S, 0);
  memset(&c->stats, 0, sizeof(c->stats));
  c->last_step = 0;
  c->stepped = false;
  if (initial_slot_expert) {
    for (int s = 0; s < c->S; ++s) {
      const int e = initial_slot_expert[s];
      if (e < -1 || e >= c->E) {
        delete c;
        return fail(MOE_ERR_INVALID_ARG, "initial slot %d holds expert %d out of range", s, e);
      }
      if (e >= 0) {
        if (c->expert_slot[e] >= 0) {
          delete c;
          return fail(MOE_ERR_INVALID_ARG, "expert %d placed twice", e);
        }
        c->slot_expert[s] = e;
        c->expert_slot[e] = s;
      }
    }
  }
  *out = c;
  return ok();
}

void moe_cache_destroy(moe_cache* cache) { delete cache; }

}  // extern "C"

// Saved state: a fixed header, then the arrays, then max_pending refill records (the first
// n_pending in planning order, the rest zero).  Little-endian plain data, no pointers.
namespace {
constexpr uint32_t kStateMagic = 0x43454F4Du;  // "MOEC"
constexpr uint32_t kStateVersion = 1;
struct StateHdr {
  uint32_t magic, version;
  int32_t E, S, K;
  moe_cache_config cfg;
  int32_t stepped, n_pending;
  int64_t last_step;
  moe_cache_stats stats;
};
struct StatePending {
  int32_t expert, slot;
  int64_t visible;
};
size_t state_bytes(int E, int S, int Q) {
  return sizeof(StateHdr) + 4 * (size_t)(S + E) + 8 * (size_t)(S + E) + sizeof(StatePending) * (size_t)Q;
}
}  // namespace

extern "C" {

moe_status moe_cache_state_bytes(const moe_cache* c, size_t* bytes) {
  if (!c || !bytes) return fail(MOE_ERR_INVALID_ARG, "moe_cache_state_bytes: NULL argument");
  *bytes = state_bytes(c->E, c->S, c->cfg.max_pending);
  return ok();
}

moe_status moe_cache_save(const moe_cache* c, void* buf, size_t bytes) {
  if (!c || !buf) return fail(MOE_ERR_INVALID_ARG, "moe_cache_save: NULL argument");
  const size_t need = state_bytes(c->E, c->S, c->cfg.max_pending);
  if (bytes < need) return fail(MOE_ERR_INVALID_ARG, "moe_cache_save: %zu bytes < %zu", bytes, need);
  uint8_t* p = static_cast<uint8_t*>(buf);
  memset(p, 0, need);
  StateHdr h;
  memset(&h, 0, sizeof(h));
  h.magic = kStateMagic;
  h.version = kStateVersion;
  h.E = c->E;
  h.S = c->S;
  h.K = c->K;
  h.cfg = c->cfg;
  h.stepped = c->stepped ? 1 : 0;
  h.n_pending = (int32_t)c->pending.size();
  h.last_step = c->last_step;
  h.stats = c->stats;
  memcpy(p, &h, sizeof(h));
  p += sizeof(h);
  memcpy(p, c->slot_expert.data(), 4 * (size_t)c->S);
  p += 4 * (size_t)c->S;
  memcpy(p, c->expert_slot.data(), 4 * (size_t)c->E);
  p += 4 * (size_t)c->E;
  memcpy(p, c->last_use.data(), 8 * (size_t)c->S);
  p += 8 * (size_t)c->S;
  memcpy(p, c->freq.data(), 8 * (size_t)c->E);
  p += 8 * (size_t)c->E;
  for (const auto& q : c->pending) {
    const StatePending r = {q.expert, q.slot, q.visible};
    memcpy(p, &r, sizeof(r));
    p += sizeof(r);
  }
  return ok();
}

moe_status moe_cache_restore(moe_cache* c, const void* buf, size_t bytes) {
  if (!c || !buf) return fail(MOE_ERR_INVALID_ARG, "moe_cache_restore: NULL argument");
  if (bytes < sizeof(StateHdr)) return fail(MOE_ERR_INVALID_ARG, "moe_cache_restore: %zu bytes hold no header", bytes);
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  StateHdr h;
  memcpy(&h, p, sizeof(h));
  if (h.magic != kStateMagic || h.version != kStateVersion)
    return fail(MOE_ERR_INVALID_ARG, "moe_cache_restore: not a saved cache state (magic %08x, version %u)",
                h.magic, h.version);
  if (h.E != c->E || h.S != c->S || h.K != c->K)
    return fail(MOE_ERR_STATE, "moe_cache_restore: state of (E=%d S=%d k=%d) into a cache of (E=%d S=%d k=%d)",
                h.E, h.S, h.K, c->E, c->S, c->K);
  const moe_cache_config& g = h.cfg;
  if ((g.policy != MOE_POLICY_LRU && g.policy != MOE_POLICY_LFRU) || g.max_refills_per_step < 0 ||
      g.lag_steps < 1 || g.max_pending < 1 || g.decay_period < 0 || h.n_pending < 0 ||
      h.n_pending > g.max_pending)
    return fail(MOE_ERR_INVALID_ARG, "moe_cache_restore: configuration out of range");
  const size_t need = state_bytes(h.E, h.S, g.max_pending);
  if (bytes < need) return fail(MOE_ERR_INVALID_ARG, "moe_cache_restore: %zu bytes < %zu", bytes, need);
  p += sizeof(h);
  std::vector<int32_t> se(h.S), es(h.E);
  std::vector<int64_t> lu(h.S), fq(h.E);
  memcpy(se.data(), p, 4 * (size_t)h.S);
  p += 4 * (size_t)h.S;
  memcpy(es.data(), p, 4 * (size_t)h.E);
  p += 4 * (size_t)h.E;
  memcpy(lu.data(), p, 8 * (size_t)h.S);
  p += 8 * (size_t)h.S;
  memcpy(fq.data(), p, 8 * (size_t)h.E);
  p += 8 * (size_t)h.E;
  std::vector<moe_cache::Pending> pend(h.n_pending);
  for (int i = 0; i < h.n_pending; ++i) {
    StatePending r;
    memcpy(&r, p + sizeof(r) * i, sizeof(r));
    pend[i] = {r.expert, r.slot, r.visible};
  }
  // the maps must be inverse of each other, in range; pending refills target empty slots
  for (int s = 0; s < h.S; ++s)
    if (se[s] < -1 || se[s] >= h.E || (se[s] >= 0 && es[se[s]] != s))
      return fail(MOE_ERR_INVALID_ARG, "moe_cache_restore: slot %d is inconsistent", s);
  for (int e = 0; e < h.E; ++e)
    if (es[e] < -1 || es[e] >= h.S || (es[e] >= 0 && se[es[e]] != e))
      return fail(MOE_ERR_INVALID_ARG, "moe_cache_restore: expert %d is inconsistent", e);
  for (const auto& q : pend)
    if (q.expert < 0 || q.expert >= h.E || q.slot < 0 || q.slot >= h.S || se[q.slot] != -1 ||
        es[q.expert] != -1)
      return fail(MOE_ERR_INVALID_ARG, "moe_cache_restore: a pending refill is inconsistent");
  c->cfg = g;
  c->slot_expert.swap(se);
  c->expert_slot.swap(es);
  c->last_use.swap(lu);
  c->freq.swap(fq);
  c->pending.swap(pend);
  c->stats = h.stats;
  c->last_step = h.last_step;
  c->stepped = h.stepped != 0;
  return ok();
}

moe_status moe_cache_policy_step(moe_cache* c, int64_t step, const int32_t* topk_ids, int32_t M,
                                 moe_refill* plan, int32_t* n_plan, int32_t* expert_to_slot,
                                 moe_cache_stats* stats) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cache is NULL");
  if (!n_plan || !expert_to_slot)
    return fail(MOE_ERR_INVALID_ARG, "n_plan and expert_to_slot are required");
  if (M < 0) return fail(MOE_ERR_INVALID_ARG, "M < 0");
  if (c->stepped && step <= c->last_step)
    return fail(MOE_ERR_STATE, "step %lld does not follow step %lld", (long long)step,
                (long long)c->last_step);
  const bool observe = topk_ids != nullptr && M > 0;
  const int n_routes = observe ? M * c->K : 0;
  for (int r = 0; r < n_routes; ++r)
    if (topk_ids[r] < 0 || topk_ids[r] >= c->E)
      return fail(MOE_ERR_INVALID_ARG, "route %d: expert %d out of range", r, topk_ids[r]);
  if (observe && !plan && c->cfg.max_refills_per_step > 0)
    return fail(MOE_ERR_INVALID_ARG, "plan is NULL");
  *n_plan = 0;
  c->stepped = true;
  c->last_step = step;

  // 1. refills that become visible now
  {
    std::vector<moe_cache::Pending> keep;
    for (const auto& p : c->pending) {
      if (p.visible <= step) {
        c->slot_expert[p.slot] = p.expert;
        c->expert_slot[p.expert] = p.slot;
      } else {
        keep.push_back(p);
      }
    }
    c->pending.swap(keep);
  }
  c->stats.steps += 1;

  if (observe) {
    // route counts of the observed step
    c->touched.clear();
    for (int r = 0; r < n_routes; ++r) {
      const int e = topk_ids[r];
      if (c->count[e]++ == 0) c->touched.push_back(e);
    }
    c->stats.routes += n_routes;
    for (int r = 0; r < n_routes; ++r)
      if (c->expert_slot[topk_ids[r]] >= 0) c->stats.hits += 1;
    if (c->cfg.policy == MOE_POLICY_LFRU) {
      if (c->cfg.decay_period > 0 && step > 0 && step % c->cfg.decay_period == 0)
        for (auto& f : c->freq) f >>= 1;
      for (int e : c->touched) c->freq[e] += c->count[e];
    }
    // 2. recency of the routed resident experts
    std::fill(c->used.begin(), c->used.end(), 0);
    for (int e : c->touched) {
      const int s = c->expert_slot[e];
      if (s >= 0) {
        c->last_use[s] = step;
        c->used[s] = 1;
      }
    }
    // 3. admissions: cold, not in flight; by (count desc, id asc)
    std::vector<int32_t> cands;
    for (int e : c->touched)
      if (c->expert_slot[e] < 0 && !expert_pending(c, e)) cands.push_back(e);
    std::sort(cands.begin(), cands.end(), [c](int a, int b) {
      return c->count[a] != c->count[b] ? c->count[a] > c->count[b] : a < b;
    });
    int admitted = 0;
    for (int e : cands) {
      if (admitted >= c->cfg.max_refills_per_step ||
          (int)c->pending.size() >= c->cfg.max_pending)
        break;
      const int v = choose_victim(c);
      if (v < 0) break;
      const int old = c->slot_expert[v];
      if (old >= 0) {
        c->expert_slot[old] = -1;
        c->stats.evictions += 1;
      }
      c->slot_expert[v] = -1;
      c->last_use[v] = step;
      const int64_t vis = step + c->cfg.lag_steps;
      c->pending.push_back({e, v, vis});
      plan[admitted].expert = e;
      plan[admitted].slot = v;
      plan[admitted].evicted = old;
      plan[admitted].reserved = 0;
      plan[admitted].visible_step = vis;
      ++admitted;
      c->stats.refills += 1;
    }
    *n_plan = admitted;
    for (int e : c->touched) c->count[e] = 0;
  }
  // 4. publish
  memcpy(expert_to_slot, c->expert_slot.data(), sizeof(int32_t) * c->E);
  if (stats) *stats = c->stats;
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// GPU-resident cache: host side (state layout, validation, launches).  The policy kernel is in
// moe_dcache.hip.
// ---------------------------------------------------------------------------------------------
static moe_status check_dcache_config(const moe_shape* shape, const moe_cache_config* cfg) {
  if (!cfg) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (cfg->policy != MOE_POLICY_LRU && cfg->policy != MOE_POLICY_LFRU)
    return fail(MOE_ERR_INVALID_ARG, "unknown policy %d", cfg->policy);
  if (cfg->max_refills_per_step < 0 || cfg->max_refills_per_step > kDcacheMaxQ ||
      cfg->lag_steps < 1 || cfg->max_pending < 1 || cfg->max_pending > kDcacheMaxQ ||
      cfg->decay_period < 0)
    return fail(MOE_ERR_INVALID_ARG,
                "device cache config out of range (R=%d in [0,%d], L=%d >= 1, Q=%d in [1,%d], decay=%d)",
                cfg->max_refills_per_step, kDcacheMaxQ, cfg->lag_steps, cfg->max_pending,
                kDcacheMaxQ, cfg->decay_period);
  (void)shape;
  return MOE_OK;
}

static moe_status check_dcache_state(const moe_shape* shape, const void* state, size_t bytes) {
  if (!state) return fail(MOE_ERR_INVALID_ARG, "device cache state is NULL");
  if (reinterpret_cast<uintptr_t>(state) & 255)
    return fail(MOE_ERR_INVALID_ARG, "device cache state must be 256-byte aligned");
  const size_t need = dcache_layout(shape->n_experts, shape->n_slots).total;
  if (bytes < need) return fail(MOE_ERR_WORKSPACE, "device cache state %zu bytes < %zu", bytes, need);
  return MOE_OK;
}

extern "C" {

moe_status moe_device_cache_size(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = dcache_layout(shape->n_experts, shape->n_slots).total;
  return ok();
}

moe_status moe_device_cache_init(const moe_shape* shape, const moe_cache_config* config,
                                 const int32_t* initial_slot_expert, int64_t first_step,
                                 void* state, size_t state_bytes, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if ((st = check_dcache_config(shape, config)) != MOE_OK) return st;
  if ((st = check_dcache_state(shape, state, state_bytes)) != MOE_OK) return st;
  const int E = shape->n_experts, S = shape->n_slots;
  const DevCacheLayout D = dcache_layout(E, S);
  std::vector<uint8_t> img(D.total, 0);
  DevCacheHdr h;
  memset(&h, 0, sizeof(h));
  h.step = first_step;
  h.E = E;
  h.S = S;
  h.R = config->max_refills_per_step;
  h.L = config->lag_steps;
  h.Q = config->max_pending;
  h.policy = config->policy;
  h.decay = config->decay_period;
  memcpy(img.data(), &h, sizeof(h));
  int32_t* se = reinterpret_cast<int32_t*>(img.data() + D.slot_expert);
  int32_t* es = reinterpret_cast<int32_t*>(img.data() + D.expert_slot);
  int64_t* lu = reinterpret_cast<int64_t*>(img.data() + D.last_use);
  for (int s = 0; s < S; ++s) {
    se[s] = -1;
    lu[s] = -1;
  }
  for (int e = 0; e < E; ++e) es[e] = -1;
  if (initial_slot_expert) {
    for (int s = 0; s < S; ++s) {
      const int e = initial_slot_expert[s];
      if (e < -1 || e >= E) return fail(MOE_ERR_INVALID_ARG, "initial slot %d holds expert %d out of range", s, e);
      if (e >= 0) {
        if (es[e] >= 0) return fail(MOE_ERR_INVALID_ARG, "expert %d placed twice", e);
        se[s] = e;
        es[e] = s;
      }
    }
  }
  hipError_t e = hipMemcpyAsync(state, img.data(), D.total, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);  // (the host image is local)
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "device cache init: %s", hipGetErrorString(e));
  return ok();
}

moe_status moe_device_cache_step(const moe_shape* shape, void* state, size_t state_bytes,
                                 const int32_t* observed_ids, int32_t n_observed,
                                 int32_t* expert_to_slot, moe_refill* plan, int32_t* n_plan,
                                 hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if ((st = check_dcache_state(shape, state, state_bytes)) != MOE_OK) return st;
  if (n_observed < 0 || n_observed > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "n_observed = %d outside [0, 2^20]", n_observed);
  if (n_observed > 0 && !observed_ids) return fail(MOE_ERR_INVALID_ARG, "observed_ids is NULL");
  if (!expert_to_slot || !plan || !n_plan)
    return fail(MOE_ERR_INVALID_ARG, "expert_to_slot, plan and n_plan are required");
  hipError_t e = launch_dcache_step(static_cast<uint8_t*>(state), shape->n_experts, shape->n_slots,
                                    observed_ids, n_observed, expert_to_slot, plan, n_plan, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "device cache step launch: %s", hipGetErrorString(e));
  return ok();
}

moe_status moe_device_cache_copy(const moe_shape* shape, const int32_t* n_plan,
                                 const moe_refill* plan, const uint8_t* host_bank, uint8_t* slots,
                                 hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!n_plan || !plan || !host_bank || !slots)
    return fail(MOE_ERR_INVALID_ARG, "moe_device_cache_copy: NULL pointer");
  if (reinterpret_cast<uintptr_t>(slots) & 255)
    return fail(MOE_ERR_INVALID_ARG, "slots must be 256-byte aligned");
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, host_bank);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();  // (a failed query leaves nothing behind)
    return fail(MOE_ERR_INVALID_ARG, "moe_device_cache_copy: host_bank is not pinned host memory");
  }
  void* dev_bank = nullptr;
  e = hipHostGetDevicePointer(&dev_bank, const_cast<uint8_t*>(host_bank), 0);
  if (e != hipSuccess || dev_bank == nullptr)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_device_cache_copy: host_bank is not pinned host memory mapped for the device (%s)",
                hipGetErrorString(e));
  if (reinterpret_cast<uintptr_t>(dev_bank) & 15)
    return fail(MOE_ERR_INVALID_ARG, "host_bank must be 16-byte aligned");
  e = launch_dcache_copy(n_plan, plan, static_cast<const uint8_t*>(dev_bank), slots,
                         expert_image_bytes(shape),
                         shape->n_experts, shape->n_slots, kDcacheMaxQ, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "device cache copy launch: %s", hipGetErrorString(e));
  return ok();
}

moe_status moe_device_cache_stats(const moe_shape* shape, const void* state, size_t state_bytes,
                                  moe_cache_stats* stats, hipStream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if ((st = check_dcache_state(shape, state, state_bytes)) != MOE_OK) return st;
  if (!stats) return fail(MOE_ERR_INVALID_ARG, "stats is NULL");
  static_assert(sizeof(moe_cache_stats) == 5 * sizeof(int64_t), "stats layout");
  hipError_t e = hipMemcpyAsync(stats, static_cast<const uint8_t*>(state) + offsetof(DevCacheHdr, stats),
                                sizeof(moe_cache_stats), hipMemcpyDefault, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
