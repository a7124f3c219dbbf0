"""Per-layer GPU slot cache policy, step by step (plain Python, small integer algorithm).

Sources (page title, section):
  * MoE expert offload (xinfer docs), "How it works": a per-layer LRU table; routed experts
    are looked up, misses get least-recently-used slots, expert ids become slot ids.
  * NInfer-Offload v0.4.0 -- expert cache, "New": experts the router keeps choosing are copied
    to the GPU in the background, at most two per layer and call, without stalling decode,
    replacing the least used ones; a static mode keeps the startup placement.
  * tinyserve -- MoE Expert Offloading for Consumer GPUs, "How it works" item 3 and
    "Configuration": frequency-recency (LFRU) eviction keyed by (layer, expert); the GPU slot
    map is synced lazily.

Readings taken where the pages are silent or disagree:
  * Refills land after a fixed lag L >= 1 steps (deterministic "background"): a refill chosen
    at step t becomes visible in the published map at step t + L.
  * The victim is evicted at once: its old expert is cold from the map published at step t.
    A miss counts as a use: the refilled slot's recency is the step that requested it.
  * Victim order: the lowest-index empty slot that is not being refilled; else, among slots
    that are resident, not being refilled and not used by the observed routes of this step,
    LRU takes the smallest (last_use, slot) and LFRU the smallest (freq, last_use, slot).
  * LFRU frequency: +1 per observed route; every ``decay_period`` steps all counts halve
    (integer shift), so the victim choice involves no floating point.
  * Miss candidates (routed, cold, not already being refilled) are admitted by route count at
    the step (descending), then expert id (ascending); at most R per step and Q in flight.

``step(t, obs_ids)`` takes the routes observed for step t (a pipeline may pass an older
step's routes; None = nothing observed), updates the state and returns the map to publish
for step t plus the refill plan.
"""
from __future__ import annotations

import numpy as np

LRU = 0
LFRU = 1


class SlotCachePolicy:
    def __init__(self, n_experts, n_slots, initial_slot_expert=None, policy=LRU,
                 max_refills=2, lag=1, max_pending=2, decay_period=64):
        if lag < 1:
            raise ValueError("lag must be >= 1")
        self.E, self.S = int(n_experts), int(n_slots)
        self.policy = policy
        self.R, self.L, self.Q = int(max_refills), int(lag), int(max_pending)
        self.decay_period = int(decay_period)
        self.slot_expert = [-1] * self.S
        self.expert_slot = [-1] * self.E
        if initial_slot_expert is not None:
            for s, e in enumerate(initial_slot_expert):
                e = int(e)
                if e >= 0:
                    if self.expert_slot[e] >= 0:
                        raise ValueError(f"expert {e} placed twice")
                    self.slot_expert[s] = e
                    self.expert_slot[e] = s
        self.last_use = [-1] * self.S
        self.freq = [0] * self.E
        self.pending = []  # (expert, slot, visible_step), in the order they were planned
        self.stats = {"steps": 0, "routes": 0, "hits": 0, "refills": 0, "evictions": 0}

    # -- victim choice ---------------------------------------------------------------------
    def _victim(self, used_slots):
        pending_slots = {s for (_, s, _) in self.pending}
        for s in range(self.S):
            if self.slot_expert[s] < 0 and s not in pending_slots:
                return s
        best, best_key = None, None
        for s in range(self.S):
            if s in pending_slots or s in used_slots or self.slot_expert[s] < 0:
                continue
            if self.policy == LFRU:
                key = (self.freq[self.slot_expert[s]], self.last_use[s], s)
            else:
                key = (self.last_use[s], s)
            if best_key is None or key < best_key:
                best, best_key = s, key
        return best

    # -- one step --------------------------------------------------------------------------
    def step(self, t: int, obs_ids=None):
        t = int(t)
        # 1. refills that become visible now
        still = []
        for (e, s, vis) in self.pending:
            if vis <= t:
                self.slot_expert[s] = e
                self.expert_slot[e] = s
            else:
                still.append((e, s, vis))
        self.pending = still
        plan = []
        self.stats["steps"] += 1
        if obs_ids is not None:
            flat = [int(v) for v in np.asarray(obs_ids).reshape(-1)]
            count = {}
            for e in flat:
                count[e] = count.get(e, 0) + 1
            self.stats["routes"] += len(flat)
            self.stats["hits"] += sum(1 for e in flat if self.expert_slot[e] >= 0)
            if self.policy == LFRU:
                if self.decay_period and t > 0 and t % self.decay_period == 0:
                    self.freq = [f >> 1 for f in self.freq]
                for e, c in count.items():
                    self.freq[e] += c
            # 2. recency of the resident experts that were routed
            used = set()
            for e in count:
                s = self.expert_slot[e]
                if s >= 0:
                    self.last_use[s] = t
                    used.add(s)
            # 3. admissions
            pending_experts = {e for (e, _, _) in self.pending}
            cands = [e for e in count if self.expert_slot[e] < 0 and e not in pending_experts]
            cands.sort(key=lambda e: (-count[e], e))
            for e in cands:
                if len(plan) >= self.R or len(self.pending) >= self.Q:
                    break
                v = self._victim(used)
                if v is None:
                    break
                old = self.slot_expert[v]
                if old >= 0:
                    self.expert_slot[old] = -1
                    self.stats["evictions"] += 1
                self.slot_expert[v] = -1
                self.last_use[v] = t  # a miss is a use: the incoming expert is the most recent
                self.pending.append((e, v, t + self.L))
                plan.append((e, v, old, t + self.L))
                self.stats["refills"] += 1
        # 4. publish
        return np.array(self.expert_slot, dtype=np.int32), plan


def simulate(policy: SlotCachePolicy, ids_per_step, readback_delay: int = 1):
    """Run a whole decode loop: at step t the policy observes the routes of step t - D.

    Returns per-step maps, plans and the cold-route count of each step's own routes under that
    step's map (what the GPU reports as skipped).
    """
    maps, plans, cold = [], [], []
    for t, ids in enumerate(ids_per_step):
        obs = ids_per_step[t - readback_delay] if t - readback_delay >= 0 else None
        m, p = policy.step(t, obs)
        maps.append(m)
        plans.append(p)
        flat = np.asarray(ids).reshape(-1)
        cold.append(int((m[flat] < 0).sum()))
    return maps, plans, cold
