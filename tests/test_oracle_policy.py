"""Pins of the oracle's slot-cache policy.

A second simulator, written independently (a recency list of slots that is reordered on use
instead of per-slot timestamps), must agree bit-exactly on random route streams; a
hand-worked trace pins the lag and eviction rules; invariants hold on every step.
"""
import numpy as np
import pytest

from oracle.cache_policy import LFRU, LRU, SlotCachePolicy, simulate


class RecencyListCache:
    """Independent formulation: a recency list of slots (least recent first) moved on use."""

    def __init__(self, E, S, init, policy, R, L, Q, decay):
        self.E, self.S, self.policy, self.R, self.L, self.Q, self.decay = E, S, policy, R, L, Q, decay
        self.recency = [s for s in range(S)]  # never-used slots first, in slot order
        self.holds = {s: int(init[s]) for s in range(S) if init[s] >= 0}  # slot -> expert
        self.never_filled = sorted(s for s in range(S) if init[s] < 0)
        self.inflight = []  # [expert, slot, visible]
        self.freq = np.zeros(E, dtype=np.int64)

    def step(self, t, obs):
        keep = []
        for e, s, vis in self.inflight:
            if vis <= t:
                self.holds[s] = e
            else:
                keep.append([e, s, vis])
        self.inflight = keep
        plan = []
        if obs is not None:
            flat = [int(v) for v in np.asarray(obs).reshape(-1)]
            uniq = sorted(set(flat))
            cnt = {e: flat.count(e) for e in uniq}
            if self.policy == LFRU:
                if self.decay and t > 0 and t % self.decay == 0:
                    self.freq >>= 1
                for e in uniq:
                    self.freq[e] += cnt[e]
            where = {e: s for s, e in self.holds.items()}
            used = sorted(where[e] for e in uniq if e in where)
            touched = list(used)
            busy_e = {f[0] for f in self.inflight}
            cands = sorted((e for e in uniq if e not in where and e not in busy_e),
                           key=lambda e: (-cnt[e], e))
            for e in cands:
                if len(plan) >= self.R or len(self.inflight) >= self.Q:
                    break
                busy_s = {f[1] for f in self.inflight}
                free = [s for s in self.never_filled if s not in busy_s]
                if free:
                    v, old = free[0], -1
                    self.never_filled.remove(v)
                else:
                    pool = [s for s in self.recency
                            if s in self.holds and s not in used and s not in busy_s]
                    if not pool:
                        break
                    if self.policy == LFRU:
                        rank = {s: i for i, s in enumerate(self.recency)}
                        v = min(pool, key=lambda s: (self.freq[self.holds[s]], rank[s]))
                    else:
                        v = pool[0]
                    old = self.holds.pop(v)
                self.inflight.append([e, v, t + self.L])
                plan.append((e, v, old, t + self.L))
                touched.append(v)
            # every slot touched at t becomes most recent, lower slot first among them
            self.recency = [s for s in self.recency if s not in touched] + sorted(touched)
        m = np.full(self.E, -1, dtype=np.int32)
        for s, e in self.holds.items():
            m[e] = s
        return m, plan


def _streams(E, k, T, seed, skew=1.2):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** skew
    p /= p.sum()
    perm = rng.permutation(E)
    out = []
    for t in range(T):
        if t % 17 == 0:
            perm = np.roll(perm, 1)
        out.append(np.stack([perm[rng.choice(E, size=k, replace=False, p=p)] for _ in range(1 + t % 3)]))
    return out


@pytest.mark.parametrize("policy", [LRU, LFRU])
@pytest.mark.parametrize("E,S,k,L,Q,R", [(32, 8, 4, 1, 2, 2), (32, 8, 4, 3, 2, 2),
                                          (16, 6, 2, 2, 4, 3), (64, 16, 6, 5, 2, 1)])
def test_policy_agrees_with_independent_simulator(policy, E, S, k, L, Q, R):
    init = np.full(S, -1)
    init[: S // 2] = np.arange(S // 2)
    a = SlotCachePolicy(E, S, init, policy=policy, max_refills=R, lag=L, max_pending=Q, decay_period=8)
    b = RecencyListCache(E, S, init, policy, R, L, Q, 8)
    ids = _streams(E, k, 150, seed=E + S + L)
    for t in range(150):
        obs = ids[t - 1] if t >= 1 else None
        ma, pa = a.step(t, obs)
        mb, pb = b.step(t, obs)
        assert np.array_equal(ma, mb), t
        assert pa == pb, t


def test_policy_invariants():
    E, S = 32, 8
    pol = SlotCachePolicy(E, S, np.arange(S), policy=LRU, max_refills=2, lag=4, max_pending=2)
    ids = _streams(E, 4, 300, seed=11)
    maps, plans, cold = simulate(pol, ids, readback_delay=2)
    for t, (m, plan) in enumerate(zip(maps, plans)):
        resident = np.flatnonzero(m >= 0)
        assert len(resident) <= S
        slots = m[resident]
        assert len(set(slots.tolist())) == len(slots)  # injective
        assert np.all((slots >= 0) & (slots < S))
        assert len(plan) <= 2
        for (e, v, old, vis) in plan:
            assert m[e] < 0 and vis == t + 4
            if old >= 0:
                assert m[old] < 0  # evicted expert is cold in the map published at t
        assert len(pol.pending) <= 2
        flat = ids[t].reshape(-1)
        assert cold[t] == int((m[flat] < 0).sum())


def test_policy_hand_worked_trace():
    # E=6, S=2, slots start with experts 0 and 1, LRU, one refill per step, lag 2, Q=1.
    pol = SlotCachePolicy(6, 2, [0, 1], policy=LRU, max_refills=1, lag=2, max_pending=1)
    m, p = pol.step(0, np.array([[0, 2]]))
    # expert 0 used -> slot 0 busy at t=0; miss 2 takes slot 1 (expert 1 evicted now)
    assert p == [(2, 1, 1, 2)]
    assert list(m) == [0, -1, -1, -1, -1, -1]
    m, p = pol.step(1, np.array([[3, 4]]))
    assert p == [] and list(m) == [0, -1, -1, -1, -1, -1]  # one refill already in flight
    m, p = pol.step(2, np.array([[3, 2]]))
    # expert 2 lands in slot 1 at t=2 and is used; miss 3 evicts slot 0 (expert 0, last use 0)
    assert p == [(3, 0, 0, 4)]
    assert list(m) == [-1, -1, 1, -1, -1, -1]
    m, p = pol.step(4, None)
    assert list(m) == [-1, -1, 1, 0, -1, -1]
    assert pol.stats == {"steps": 4, "routes": 6, "hits": 2, "refills": 2, "evictions": 2}


def test_simulate_hand_worked_readback_trace():
    """simulate() with a readback delay of 2 steps, worked by hand (E=4, S=2, slots start with
    experts 0 and 1, LRU, one refill per step, lag 1, one in flight; one route per step).

    routes: t0 -> 2, t1 -> 3, t2 -> 0, t3 -> 2, t4 -> 1
    t0, t1: nothing observed yet; map {0:0, 1:1}; routes 2 and 3 are cold.
    t2: observes t0's route (2): miss; no empty slot, both slots unused since the start, LRU
        (last use -1, -1) takes slot 0: expert 0 is evicted now, 2 arrives at t3.
        Map {1:1}; t2's own route (0) is cold.
    t3: 2 lands in slot 0.  Observes t1's route (3): miss; slot 0 was last used at t2 (the
        refill), slot 1 never: slot 1, expert 1 evicted, 3 arrives at t4.  Map {2:0}; route 2 hot.
    t4: 3 lands in slot 1.  Observes t2's route (0): miss; slot 0 (last use 2) is older than
        slot 1 (3): expert 2 evicted, 0 arrives at t5.  Map {3:1}; route 1 is cold.
    A delay of 1 instead of 2 changes the plan at t1 already.
    """
    ids = [np.array([[e]]) for e in (2, 3, 0, 2, 1)]
    pol = SlotCachePolicy(4, 2, [0, 1], policy=LRU, max_refills=1, lag=1, max_pending=1)
    maps, plans, cold = simulate(pol, ids, readback_delay=2)
    assert [list(m) for m in maps] == [[0, 1, -1, -1], [0, 1, -1, -1], [-1, 1, -1, -1],
                                       [-1, -1, 0, -1], [-1, -1, -1, 1]]
    assert plans == [[], [], [(2, 0, 0, 3)], [(3, 1, 1, 4)], [(0, 0, 2, 5)]]
    assert cold == [1, 1, 1, 0, 1]
    pol1 = SlotCachePolicy(4, 2, [0, 1], policy=LRU, max_refills=1, lag=1, max_pending=1)
    _, plans1, _ = simulate(pol1, ids, readback_delay=1)
    assert plans1[1] == [(2, 0, 0, 2)]
