// GPU-resident slot cache: the per-layer slot-cache policy as a kernel over state kept in
// device memory, and a fixed-shape kernel that copies the planned experts from device-mapped
// pinned host memory into their slots [MoE expert offload, "How it works", Decode: the LRU table
// is kept on the GPU, a kernel assigns slots to misses and a second kernel copies the missing
// experts straight from device-mapped pinned host memory; both have fixed launch shapes and read
// the miss count from device memory, so decode stays inside graphs with no host sync].
//
// The policy is the one of moe_cache_policy_step (moe_cache.cpp), step for step, so that the
// two and the oracle's replay agree bit for bit: visible refills land, the observed routes update
// the counters, recency (and LFRU frequencies), routed cold experts are admitted by (route count
// descending, id ascending) while fewer than R were admitted and fewer than Q are in flight,
// each into the lowest empty slot or the least recently used (LFRU: least frequent, then least
// recent) slot not routed at the step and not in flight; the evicted expert is cold at once and
// the new one visible L steps later; then the map is published.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace {

// The largest of a 64-bit value over the wave (every lane gets it).
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, off);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ uint64_t wave_min64(uint64_t v) { return ~wave_max64(~v); }
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

}  // namespace

// One step of the policy, by one wave.  obs: n_obs observed route ids (ids outside [0, E) are not
// observed; with none observed the step only lands visible refills and publishes the map).
// Outputs: map_out [E], plan [R], *n_plan.
__global__ __launch_bounds__(64) void k_dcache_step(uint8_t* __restrict__ state,
                                                    const int32_t* __restrict__ obs, int n_obs,
                                                    int32_t* __restrict__ map_out,
                                                    moe_refill* __restrict__ plan,
                                                    int32_t* __restrict__ n_plan) {
  __shared__ DevCacheHdr h;
  extern __shared__ __align__(16) uint8_t sm[];
  const int lane = threadIdx.x;
  DevCacheHdr* gh = reinterpret_cast<DevCacheHdr*>(state);
  if (lane == 0) h = *gh;
  __syncthreads();
  const int E = h.E, S = h.S;
  const DevCacheLayout D = dcache_layout(E, S);
  int32_t* g_se = reinterpret_cast<int32_t*>(state + D.slot_expert);
  int32_t* g_es = reinterpret_cast<int32_t*>(state + D.expert_slot);
  int64_t* g_lu = reinterpret_cast<int64_t*>(state + D.last_use);
  int64_t* g_fq = reinterpret_cast<int64_t*>(state + D.freq);
  // LDS copies: last_use [S], freq [E] (8-byte), slot_expert [S], expert_slot [E], used [S],
  // count [E]
  int64_t* lu = reinterpret_cast<int64_t*>(sm);
  int64_t* fq = lu + S;
  int32_t* se = reinterpret_cast<int32_t*>(fq + E);
  int32_t* es = se + S;
  int32_t* used = es + E;
  int32_t* cnt = used + S;
  for (int i = lane; i < S; i += 64) {
    se[i] = g_se[i];
    lu[i] = g_lu[i];
    used[i] = 0;
  }
  for (int i = lane; i < E; i += 64) {
    es[i] = g_es[i];
    fq[i] = g_fq[i];
    cnt[i] = 0;
  }
  __syncthreads();
  const int64_t t = h.step;
  // 1. refills that become visible now (in planning order)
  if (lane == 0) {
    int keep = 0;
    for (int i = 0; i < h.n_pending; ++i) {
      if (h.pend_vis[i] <= t) {
        se[h.pend_s[i]] = h.pend_e[i];
        es[h.pend_e[i]] = h.pend_s[i];
      } else {
        h.pend_e[keep] = h.pend_e[i];
        h.pend_s[keep] = h.pend_s[i];
        h.pend_vis[keep] = h.pend_vis[i];
        ++keep;
      }
    }
    h.n_pending = keep;
    h.stats[0] += 1;  // steps
  }
  __syncthreads();
  int admitted = 0;
  // 2. the observed routes: counts, route and hit counters
  int nvalid = 0, nhit = 0;
  for (int r = lane; r < n_obs; r += 64) {
    const int e = obs[r];
    if (e >= 0 && e < E) {
      atomicAdd(&cnt[e], 1);
      ++nvalid;
      nhit += es[e] >= 0 ? 1 : 0;
    }
  }
  nvalid = wave_sum_i(nvalid);
  nhit = wave_sum_i(nhit);
  __syncthreads();
  if (nvalid > 0) {
    if (lane == 0) {
      h.stats[1] += nvalid;  // routes
      h.stats[2] += nhit;    // hits
    }
    if (h.policy == MOE_POLICY_LFRU) {
      const bool decay = h.decay > 0 && t > 0 && t % h.decay == 0;
      for (int e = lane; e < E; e += 64) fq[e] = (decay ? fq[e] >> 1 : fq[e]) + cnt[e];
    }
    // 3. recency of the routed resident experts
    for (int e = lane; e < E; e += 64)
      if (cnt[e] > 0 && es[e] >= 0) {
        lu[es[e]] = t;
        used[es[e]] = 1;
      }
    __syncthreads();
    // 4. admissions, best candidate first: (count descending, id ascending)
    for (int a = 0; a < h.R; ++a) {
      if (h.n_pending >= h.Q) break;
      uint64_t best = 0;
      for (int e = lane; e < E; e += 64) {
        bool pend = false;
        for (int i = 0; i < h.n_pending; ++i) pend = pend || h.pend_e[i] == e;
        if (cnt[e] > 0 && es[e] < 0 && !pend)
        {
          const uint64_t key = ((uint64_t)cnt[e] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
          best = key > best ? key : best;
        }
      }
      best = wave_max64(best);
      if (best == 0) break;
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
      // victim: the lowest empty slot not in flight ...
      uint64_t vmin = ~0ull;
      for (int s = lane; s < S; s += 64) {
        bool pend = false;
        for (int i = 0; i < h.n_pending; ++i) pend = pend || h.pend_s[i] == s;
        if (se[s] < 0 && !pend && (uint64_t)s < vmin) vmin = (uint64_t)s;
      }
      vmin = wave_min64(vmin);
      if (vmin == ~0ull) {
        // ... else the smallest (freq [LFRU], last use, slot) among resident slots that are
        // neither routed at this step nor in flight
        uint64_t kf = ~0ull, kl = ~0ull;
        for (int pass = 0; pass < 3; ++pass) {
          uint64_t m = ~0ull;
          for (int s = lane; s < S; s += 64) {
            bool pend = false;
            for (int i = 0; i < h.n_pending; ++i) pend = pend || h.pend_s[i] == s;
            if (se[s] < 0 || used[s] || pend) continue;
            const uint64_t f = h.policy == MOE_POLICY_LFRU ? (uint64_t)fq[se[s]] : 0ull;
            const uint64_t l = (uint64_t)(lu[s] + 1);  // last use >= -1
            uint64_t c = ~0ull;
            if (pass == 0) c = f;
            else if (pass == 1 && f == kf) c = l;
            else if (pass == 2 && f == kf && l == kl) c = (uint64_t)s;
            m = c < m ? c : m;
          }
          m = wave_min64(m);
          if (pass == 0) kf = m;
          else if (pass == 1) kl = m;
          else vmin = m;
          if (m == ~0ull) break;
        }
      }
      if (vmin == ~0ull) break;  // no victim
      const int v = (int)vmin;
      if (lane == 0) {
        const int old = se[v];
        if (old >= 0) {
          es[old] = -1;
          h.stats[4] += 1;  // evictions
        }
        se[v] = -1;
        lu[v] = t;
        h.pend_e[h.n_pending] = e;
        h.pend_s[h.n_pending] = v;
        h.pend_vis[h.n_pending] = t + h.L;
        h.n_pending += 1;
        h.stats[3] += 1;  // refills
        moe_refill rf;
        rf.expert = e;
        rf.slot = v;
        rf.evicted = old;
        rf.reserved = 0;
        rf.visible_step = t + h.L;
        plan[a] = rf;
      }
      ++admitted;
      __syncthreads();
    }
  }
  __syncthreads();
  // 5. publish the map; keep the state
  for (int e = lane; e < E; e += 64) {
    map_out[e] = es[e];
    g_es[e] = es[e];
    g_fq[e] = fq[e];
  }
  for (int s = lane; s < S; s += 64) {
    g_se[s] = se[s];
    g_lu[s] = lu[s];
  }
  if (lane == 0) {
    h.step = t + 1;
    *gh = h;
    *n_plan = admitted;
  }
}

// The planned refills: plan[0 .. *n_plan) images from the device-mapped host bank into their
// slots, 64 bytes a thread per round over the whole grid (fixed shape; nothing to do when the
// plan is empty).  Entries outside [0, E) x [0, S) are skipped.
__global__ __launch_bounds__(256) void k_dcache_copy(const int32_t* __restrict__ n_plan,
                                                     const moe_refill* __restrict__ plan,
                                                     const uint8_t* __restrict__ bank,
                                                     uint8_t* __restrict__ slots, size_t image_bytes,
                                                     int E, int S, int R) {
  const int n = min(*n_plan, R);
  const size_t chunks = image_bytes / 64;  // images are multiples of 256 bytes
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (int i = 0; i < n; ++i) {
    const moe_refill rf = plan[i];
    if (rf.expert < 0 || rf.expert >= E || rf.slot < 0 || rf.slot >= S) continue;
    const uint4* src = reinterpret_cast<const uint4*>(bank + (size_t)rf.expert * image_bytes);
    uint4* dst = reinterpret_cast<uint4*>(slots + (size_t)rf.slot * image_bytes);
    for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += stride) {
      const uint4 a = src[4 * c], b = src[4 * c + 1], d = src[4 * c + 2], f = src[4 * c + 3];
      dst[4 * c] = a;
      dst[4 * c + 1] = b;
      dst[4 * c + 2] = d;
      dst[4 * c + 3] = f;
    }
  }
}

hipError_t launch_dcache_step(uint8_t* state, int E, int S, const int32_t* obs, int n_obs,
                              int32_t* map_out, moe_refill* plan, int32_t* n_plan, hipStream_t s) {
  const size_t lds = (size_t)(S + E) * 8 + (size_t)(2 * S + 2 * E) * 4;
  hipLaunchKernelGGL(k_dcache_step, dim3(1), dim3(64), lds, s, state, obs, n_obs, map_out, plan,
                     n_plan);
  return hipGetLastError();
}

hipError_t launch_dcache_copy(const int32_t* n_plan, const moe_refill* plan, const uint8_t* bank,
                              uint8_t* slots, size_t image_bytes, int E, int S, int R,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_dcache_copy, dim3(kDcacheCopyGroups), dim3(256), 0, s, n_plan, plan, bank,
                     slots, image_bytes, E, S, R);
  return hipGetLastError();
}

}  // namespace moe
