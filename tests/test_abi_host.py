"""The C ABI without a GPU: every declared symbol is exported, the host-only calls (image
packing, cache policy, argument checks) behave as documented.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import synthetic
from expert_offloaded_routed_amd import binding as B
from oracle.cache_policy import LFRU, LRU, SlotCachePolicy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return B.load()


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:moe_status|void|const char\*)\s+(moe_\w+)\s*\(", text, re.M)
    return names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    names = _declared_functions()
    assert set(names) >= {"moe_route", "moe_experts_forward", "moe_bucket_routes", "moe_slot_refill",
                          "moe_cache_create", "moe_cache_policy_step", "moe_cache_destroy",
                          "moe_pack_expert", "moe_unpack_expert", "moe_expert_image_bytes",
                          "moe_workspace_size", "moe_layer_forward", "moe_last_error",
                          "moe_experts_gateup", "moe_experts_down", "moe_layer_forward_marked",
                          "moe_residual_bf16", "moe_layer_launches", "moe_layer_forward_residual"}
    for n in names:
        assert hasattr(lib, n), n
    # no torch in the exported signatures: the header includes only C/HIP headers
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert "torch" not in hdr and "at::" not in hdr


def test_layer_launch_counts():
    """One GPT-OSS-20B-shaped token: one fused launch with the router inside (on a GPU); a few
    tokens (at most 64 routes over at most 64 experts, or one token): router, gate/up, down;
    other calls below 64 tokens add the top-k / bucketing kernel; from 64 tokens the grouped GEMM path (top-k /
    bucketing, gate/up, down, combine after the router).  More K groups per gate/up wave than
    the fused kernel holds (H = 8192) keep three launches."""
    _lib()
    if os.environ.get("MOE_DECODE_UNFUSED") == "1":
        pytest.skip("fused decode switched off in this environment")
    g = B.make_shape(2880, 2880, 32, 4, 32)
    # M = 1 fuses only where the device can hold the whole fused grid at once (one launch, the
    # router inside, on an MI355X; 3 without a device)
    assert B.moe_layer_launches(g, 1) in (1, 3)
    assert [B.moe_layer_launches(g, M) for M in (0, 2, 16, 17, 64)] == [1, 3, 3, 4, 5]
    e512 = B.make_shape(2048, 512, 512, 10, 256)
    # one token of the E = 512 layer: router + the fused launch where the grid fits (else 3)
    assert B.moe_layer_launches(e512, 1) in (2, 3)
    assert [B.moe_layer_launches(e512, M) for M in (2, 63, 64)] == [4, 4, 5]
    assert B.moe_layer_launches(B.make_shape(8192, 512, 8, 2, 8), 1) == 3
    with pytest.raises(B.MoeError):
        B.moe_layer_launches(g, -1)


@pytest.mark.parametrize("name", ["tiny", "gptoss20b_decode", "e512_verify_stack"])
def test_pack_unpack_round_trip(name):
    _lib()
    wl = synthetic.WORKLOADS[name]
    shape = B.make_shape(wl.hidden, wl.inter, wl.n_experts, wl.top_k, wl.n_slots)
    ex = synthetic.expert_canonical(wl, 0, 1)
    img = B.moe_pack_expert(shape, ex)
    assert img.size == B.moe_expert_image_bytes(shape) and img.size % 256 == 0
    back = B.moe_unpack_expert(shape, img)
    for k, v in ex.items():
        assert np.array_equal(back[k], v), k
    # the image holds each code byte exactly once plus padding scale bytes only
    alg = sum(v.nbytes for v in ex.values())
    assert alg <= img.size <= alg * 1.01 + 256


def test_pack_layout_lane_order():
    _lib()
    shape = B.make_shape(64, 32, 2, 1, 2)
    H, I = 64, 32
    ex = {"gate_codes": np.zeros((I, H // 2), np.uint8), "gate_scales": np.full((I, 2), 120, np.uint8),
          "up_codes": np.zeros((I, H // 2), np.uint8), "up_scales": np.full((I, 2), 121, np.uint8),
          "down_codes": np.zeros((H, I // 2), np.uint8), "down_scales": np.full((H, 1), 122, np.uint8)}
    ex["gate_codes"][5, 16:32] = np.arange(16)      # gate row 5, block 1
    ex["up_codes"][7, 0:16] = np.arange(16) + 100   # up row 7, block 0
    img = B.moe_pack_expert(shape, ex)
    # gate/up tile 0: block b, lane l at (b*64 + l)*16; lanes 32.. are the up rows
    assert np.array_equal(img[(1 * 64 + 5) * 16:(1 * 64 + 5) * 16 + 16], np.arange(16))
    assert np.array_equal(img[(0 * 64 + 39) * 16:(0 * 64 + 39) * 16 + 16], np.arange(16) + 100)
    # scales after the 2 code blocks: one group, lane word, bytes = blocks 0,1 then padding 127
    s0 = 2 * 1024
    assert list(img[s0 + 5 * 4: s0 + 5 * 4 + 4]) == [120, 120, 127, 127]
    assert list(img[s0 + 39 * 4: s0 + 39 * 4 + 4]) == [121, 121, 127, 127]


def _cache_pair(policy, E=32, S=8, k=4, R=2, L=3, Q=2, decay=8):
    shape = B.make_shape(256, 512, E, k, S)
    init = np.arange(S, dtype=np.int32)
    init[-2:] = -1
    lib_cache = B.MoeCache(shape, policy=policy, max_refills_per_step=R, lag_steps=L, max_pending=Q,
                           decay_period=decay, initial_slot_expert=init)
    ref = SlotCachePolicy(E, S, init, policy=policy, max_refills=R, lag=L, max_pending=Q,
                          decay_period=decay)
    return lib_cache, ref


@pytest.mark.parametrize("policy", [LRU, LFRU])
@pytest.mark.parametrize("L,Q,R", [(1, 2, 2), (3, 2, 2), (5, 4, 3), (2, 1, 1)])
def test_host_policy_matches_oracle(policy, L, Q, R):
    _lib()
    E, S, k = 32, 8, 4
    lib_cache, ref = _cache_pair(policy, E, S, k, R, L, Q)
    rng = np.random.default_rng(L * 10 + Q + policy)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    perm = rng.permutation(E)
    for t in range(200):
        if t % 32 == 0:
            perm = np.roll(perm, 1)
        M = 1 + (t % 3)
        ids = np.stack([perm[rng.choice(E, size=k, replace=False, p=p)] for _ in range(M)]).astype(np.int32)
        obs = None if t % 7 == 3 else ids
        m_lib, plan_lib, stats = lib_cache.moe_cache_policy_step(t, obs)
        m_ref, plan_ref = ref.step(t, obs)
        assert np.array_equal(m_lib, m_ref), t
        assert plan_lib == plan_ref, t
        assert stats == ref.stats, t
    lib_cache.close()


def test_host_policy_errors():
    _lib()
    shape = B.make_shape(256, 512, 8, 2, 4)
    c = B.MoeCache(shape, initial_slot_expert=[0, 1, 2, 3])
    c.moe_cache_policy_step(5, np.array([[0, 1]]))
    with pytest.raises(B.MoeError) as e:
        c.moe_cache_policy_step(5, np.array([[0, 1]]))
    assert e.value.status == B.MOE_ERR_STATE
    with pytest.raises(B.MoeError) as e:
        c.moe_cache_policy_step(6, np.array([[0, 9]]))
    assert e.value.status == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError):
        B.MoeCache(shape, initial_slot_expert=[0, 0, 1, 2])
    with pytest.raises(B.MoeError):
        B.MoeCache(shape, lag_steps=0)


def test_argument_checks_return_status_before_any_launch():
    lib = _lib()
    good = B.make_shape(2880, 2880, 32, 4, 32)
    out = ctypes.c_size_t(0)
    for bad, code in ((B.make_shape(2880, 2880, 32, 4, 0), B.MOE_ERR_INVALID_ARG),
                      (B.make_shape(2880 + 32, 2880, 32, 4, 32), B.MOE_ERR_UNSUPPORTED),
                      (B.make_shape(2880, 2880 + 16, 32, 4, 32), B.MOE_ERR_UNSUPPORTED),
                      (B.make_shape(2880, 2880, 2048, 4, 32), B.MOE_ERR_UNSUPPORTED),
                      (B.make_shape(2880, 2880, 32, 33, 32), B.MOE_ERR_UNSUPPORTED),
                      (B.make_shape(2880, 4096 + 32, 32, 4, 32), B.MOE_ERR_UNSUPPORTED),
                      (B.make_shape(2880, 2880, 3, 4, 32), B.MOE_ERR_UNSUPPORTED)):
        assert lib.moe_expert_image_bytes(ctypes.byref(bad), ctypes.byref(out)) == code
        assert B.moe_last_error() != ""
    assert lib.moe_workspace_size(ctypes.byref(good), 1, ctypes.byref(out)) == B.MOE_OK
    need = out.value
    # undersized / misaligned / NULL workspaces are refused on the host
    assert lib.moe_route(ctypes.byref(good), 16, 1, 16, None, 16, 16, 256, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(good), 16, 1, 16, None, 16, 16, 257, need, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(good), 16, 1, 16, None, 16, 16, None, need, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(good), 16, -1, 16, None, 16, 16, 256, need, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(good), None, 1, 16, None, 16, 16, 256, need, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_experts_forward(ctypes.byref(good), 16, 1, 16, 16, None, 260, 16, None, None,
                                   256, need, None) == B.MOE_ERR_INVALID_ARG  # slots misaligned
    ident = B.make_shape(2880, 2880, 32, 4, 8)  # identity map impossible with 8 slots
    lib.moe_workspace_size(ctypes.byref(ident), 4, ctypes.byref(out))
    assert lib.moe_bucket_routes(ctypes.byref(ident), 16, 1, None, None, None, None, None, None,
                                 256, out.value, None) == B.MOE_ERR_INVALID_ARG
    experts = np.array([0, 40], np.int32)
    slots = np.array([0, 1], np.int32)
    assert lib.moe_slot_refill(ctypes.byref(good), 256, 256, experts.ctypes.data, slots.ctypes.data, 2,
                               None, None, None) == B.MOE_ERR_INVALID_ARG
    slots2 = np.array([3, 3], np.int32)
    experts2 = np.array([0, 1], np.int32)
    assert lib.moe_slot_refill(ctypes.byref(good), 256, 256, experts2.ctypes.data, slots2.ctypes.data, 2,
                               None, None, None) == B.MOE_ERR_INVALID_ARG


def test_pack_down_layout_mfma_steps_and_partial_step():
    """Down rows of a 2880-wide intermediate in 16-row tiles: 23 K steps of 4 blocks, lane l
    holding row l%16, block 4s + l/16; the last step partial (90 = 22*4 + 2 blocks, only its
    first 32 lanes stored).  Check where one block, one scale byte and the padding land."""
    _lib()
    H, I = 64, 2880
    shape = B.make_shape(H, I, 2, 1, 2)
    rng = np.random.default_rng(0)
    ex = {"gate_codes": rng.integers(0, 256, (I, H // 2), dtype=np.uint8),
          "gate_scales": rng.integers(100, 140, (I, H // 32), dtype=np.uint8),
          "up_codes": rng.integers(0, 256, (I, H // 2), dtype=np.uint8),
          "up_scales": rng.integers(100, 140, (I, H // 32), dtype=np.uint8),
          "down_codes": rng.integers(0, 256, (H, I // 2), dtype=np.uint8),
          "down_scales": rng.integers(100, 140, (H, I // 32), dtype=np.uint8)}
    img = B.moe_pack_expert(shape, ex)
    gu_tile = 2 * 1024 + 1 * 256            # H=64: 2 blocks, 1 scale group per tile
    gu_bytes = gu_tile * (I // 32)
    code_bytes = 22 * 1024 + 2 * 256        # 22 full steps, then 2 blocks x 16 rows
    dn_tile = code_bytes + 6 * 256          # ceil(23 / 4) scale words per lane
    assert img.size == -(-(gu_bytes + dn_tile * (H // 16)) // 256) * 256
    # row 21 = tile 1, row 5 of it; block 43 = step 10, lane group 3: lane 53
    t1 = gu_bytes + 1 * dn_tile
    off = t1 + (10 * 64 + 53) * 16
    assert np.array_equal(img[off:off + 16], ex["down_codes"][21, 43 * 16:44 * 16])
    # block 89 = step 22 (partial), lane group 1: lane 21 of the stored part
    off = t1 + (22 * 64 + 21) * 16
    assert np.array_equal(img[off:off + 16], ex["down_codes"][21, 89 * 16:90 * 16])
    # scale of block 43 (step 10 -> word 2, byte 2) of lane 53
    assert img[t1 + code_bytes + (2 * 64 + 53) * 4 + 2] == ex["down_scales"][21, 43]
    # block 90 (step 22, lane group 2) and step 23 do not exist: padding 127
    assert img[t1 + code_bytes + (5 * 64 + 37) * 4 + 2] == 127
    assert img[t1 + code_bytes + (5 * 64 + 5) * 4 + 3] == 127


@pytest.mark.parametrize("fmt", ["bf16", "fp8_block", "nvfp4"])
def test_other_formats_pack_round_trip_and_host_checks(fmt):
    """Images of the other formats hold the six canonical arrays row-major, each at a multiple
    of 256 bytes; the host checks of the format field run before anything is enqueued."""
    _lib()
    wl = synthetic.WORKLOADS["tiny"]
    H, I = wl.hidden, wl.inter
    shape = B.make_shape(H, I, wl.n_experts, wl.top_k, wl.n_experts, fmt)
    ex = synthetic.expert_canonical(wl, 0, 2, fmt)

    def sz(n, k):
        el = {"bf16": 2 * n * k, "fp8_block": n * k, "nvfp4": n * k // 2}[fmt]
        sc = {"bf16": 0, "fp8_block": 4 * ((n + 127) // 128) * ((k + 127) // 128),
              "nvfp4": 4 + n * (k // 16)}[fmt]
        r = lambda v: (v + 255) // 256 * 256
        return r(el) + r(sc)

    assert B.moe_expert_image_bytes(shape) == 2 * sz(I, H) + sz(H, I)
    img = B.moe_pack_expert(shape, ex)
    back = B.moe_unpack_expert(shape, img)
    for key, v in ex.items():
        if key != "format":
            assert np.array_equal(np.asarray(back[key]), np.asarray(v)), key
    # the gate elements open the image, row-major
    first = np.asarray(ex["gate_codes"]).reshape(-1)[:8]
    assert np.array_equal(img[:first.nbytes], first.view(np.uint8))
    # every format but MXFP4: router, top-k / bucketing, gate/up, down
    assert [B.moe_layer_launches(shape, M) for M in (0, 1, 64)] == [1, 4, 4]
    # the host expert path reads MXFP4 images only
    M = 1
    y = np.zeros((M, H), np.float32)
    with pytest.raises(B.MoeError) as e:
        B.moe_cold_forward_host(shape, np.zeros((wl.n_experts, B.moe_expert_image_bytes(shape)), np.uint8),
                                synthetic.activations(wl, M, 0), M, np.zeros((M, wl.top_k), np.int32),
                                np.ones((M, wl.top_k), np.float32), None, y)
    assert e.value.status == B.MOE_ERR_UNSUPPORTED


def test_unknown_format_is_rejected():
    _lib()
    for f in (-1, 4):
        with pytest.raises(B.MoeError) as e:
            B.moe_expert_image_bytes(B.make_shape(256, 512, 8, 2, 8, f))
        assert e.value.status == B.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("policy", [LRU, LFRU])
def test_host_cache_save_restore_replays_bit_exact(policy):
    """A cache restored from a state saved at step t0 (into a fresh cache created with another
    configuration) plans exactly what the original planned from t0 on, and matches the oracle;
    broken or foreign states are refused and leave the cache as it was."""
    _lib()
    E, S, k = 32, 8, 4
    orig, ref = _cache_pair(policy, E, S, k, 2, 3, 3)
    rng = np.random.default_rng(17 + policy)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    steps = [np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(1 + t % 2)]).astype(np.int32)
             for t in range(120)]
    t0, saved, tail = 70, None, []
    for t, ids in enumerate(steps):
        if t == t0:
            saved = orig.moe_cache_save()
        out = orig.moe_cache_policy_step(t, ids)
        m_ref, plan_ref = ref.step(t, ids)
        assert np.array_equal(out[0], m_ref) and out[1] == plan_ref
        if t >= t0:
            tail.append(out)
    fresh = B.MoeCache(B.make_shape(256, 512, E, k, S), policy=LRU, max_refills_per_step=1,
                       lag_steps=1, max_pending=1)
    fresh.moe_cache_restore(saved)
    for t in range(t0, len(steps)):
        m, plan, stats = fresh.moe_cache_policy_step(t, steps[t])
        m0, plan0, stats0 = tail[t - t0]
        assert np.array_equal(m, m0) and plan == plan0 and stats == stats0, t
    # the state round-trips byte for byte
    assert np.array_equal(fresh.moe_cache_save(), orig.moe_cache_save())
    # refused: not a state, truncated, inconsistent, another shape; the cache stays as it was
    before = fresh.moe_cache_save()
    bad = saved.copy()
    bad[0] ^= 0xFF
    for b in (bad, saved[:40]):
        with pytest.raises(B.MoeError) as e:
            fresh.moe_cache_restore(b)
        assert e.value.status == B.MOE_ERR_INVALID_ARG
    bad = saved.copy()
    hdr = 4 * 10 + 4 + 4 + 8 + 8 * 5  # header bytes: magic .. stats
    bad[hdr:hdr + 4] = np.frombuffer(np.int32(E + 3).tobytes(), np.uint8)  # slot 0 -> expert E+3
    with pytest.raises(B.MoeError) as e:
        fresh.moe_cache_restore(bad)
    assert e.value.status == B.MOE_ERR_INVALID_ARG
    other = B.MoeCache(B.make_shape(256, 512, E, k, S + 1))
    with pytest.raises(B.MoeError) as e:
        other.moe_cache_restore(saved)
    assert e.value.status == B.MOE_ERR_STATE
    assert np.array_equal(fresh.moe_cache_save(), before)
    for c in (orig, fresh, other):
        c.close()
