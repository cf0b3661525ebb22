"""CPU tests of the expert cache's host logic (seedmm_cache_init / plan / reset / stats):
the slot planner against an independent model of least-recently-used replacement, its
invariants, and its argument errors.  No GPU: the planner touches no device memory, so
the device and host-stream addresses below are never dereferenced."""
import ctypes

import numpy as np
import pytest

FAKE_DEV = 0x10000000     # 256-byte aligned, never dereferenced by init / plan
FAKE_HOST = 0x20000000


@pytest.fixture(scope="module")
def L():
    from pseudo_random_weight_amd import seedmm
    return seedmm


class Cache:
    def __init__(self, seedmm, E, S, H=64, I=32, P=4):
        self.sm, self.E, self.S = seedmm, E, S
        lib = seedmm.lib()
        n = lib.seedmm_cache_state_bytes(E, S)
        assert n > 0
        self.state = (ctypes.c_uint64 * ((n + 7) // 8))()
        ndev = lib.seedmm_cache_device_bytes(E, H, I, P, S)
        assert ndev > 0
        st = lib.seedmm_cache_init(ctypes.addressof(self.state), n, E, H, I, P, S,
                                   ctypes.c_void_p(FAKE_HOST), ctypes.c_void_p(FAKE_DEV),
                                   ctypes.c_void_p(FAKE_DEV), ndev)
        assert st == 0, st

    @property
    def h(self):
        return ctypes.c_void_p(ctypes.addressof(self.state))

    def plan(self, ids):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        loads = np.full(2 * self.S, -7, dtype=np.int32)
        n = ctypes.c_int(-1)
        st = self.sm.lib().seedmm_cache_plan(self.h, ids.ctypes.data_as(ctypes.c_void_p),
                                             ids.shape[0], ids.shape[1],
                                             loads.ctypes.data_as(ctypes.c_void_p),
                                             ctypes.byref(n))
        if st != 0:
            return st, None
        return 0, [(int(loads[2 * i]), int(loads[2 * i + 1])) for i in range(n.value)]

    def stats(self):
        out = (ctypes.c_uint64 * 5)()
        assert self.sm.lib().seedmm_cache_stats(self.h, out) == 0
        return list(out)


class ModelLRU:
    """Least recently used replacement as documented for seedmm_cache_plan, written out
    with Python containers: hits refresh their slot first; misses in increasing expert
    order take the lowest free slot, else the slot used longest ago (lowest on ties) that
    this call does not use."""

    def __init__(self, S):
        self.S, self.where, self.owner, self.age, self.t = S, {}, [None] * S, [0] * S, 0

    def plan(self, ids):
        want = sorted(set(int(v) for v in np.asarray(ids).ravel()))
        if len(want) > self.S:
            return None
        self.t += 1
        for e in want:
            if e in self.where:
                self.age[self.where[e]] = self.t
        out = []
        for e in want:
            if e in self.where:
                continue
            free = [s for s in range(self.S) if self.owner[s] is None]
            if free:
                v = free[0]
            else:
                v = min((s for s in range(self.S) if self.age[s] < self.t),
                        key=lambda s: (self.age[s], s))
                del self.where[self.owner[v]]
            self.owner[v], self.where[e], self.age[v] = e, v, self.t
            out.append((e, v))
        return out


@pytest.mark.parametrize("E,S,T,k,skew", [(16, 5, 1, 2, False), (100, 33, 1, 8, False),
                                          (100, 33, 3, 8, True), (40, 40, 4, 4, False),
                                          (64, 12, 2, 6, True)])
def test_plan_follows_least_recently_used(L, E, S, T, k, skew):
    rng = np.random.default_rng(E * 1000 + S)
    c, m = Cache(L, E, S), ModelLRU(S)
    hot = rng.permutation(E)[: max(k, E // 3)]
    calls = hits = misses = uses = 0
    for step in range(300):
        ids = np.empty((T, k), dtype=np.int32)
        for t in range(T):
            pool = hot if (skew and rng.random() < 0.85) else np.arange(E)
            ids[t] = rng.choice(pool, size=k, replace=False)
        want = m.plan(ids)
        st, got = c.plan(ids)
        if want is None:
            assert st == L.ECAPACITY
            continue
        assert st == 0 and got == want, step
        distinct = len(set(ids.ravel().tolist()))
        calls, uses, misses = calls + 1, uses + distinct, misses + len(got)
        hits += distinct - len(got)
        # every expert of the call is resident, in a distinct slot
        assert len(m.where) <= S
        assert all(int(e) in m.where for e in ids.ravel())
    s = c.stats()
    assert s[:4] == [calls, uses, hits, misses]
    assert s[4] == misses * L.lib().seedmm_cache_record_layout(64, 32, 4, None)


def test_plan_rejects_without_changing_state(L):
    c = Cache(L, 10, 3)
    assert c.plan([[0, 1]])[0] == 0
    before = c.stats()
    assert c.plan([[0, 10]])[0] == L.EINVAL          # id out of range
    assert c.plan([[-1, 2]])[0] == L.EINVAL
    assert c.plan([[4, 5], [6, 7]])[0] == L.ECAPACITY  # 4 distinct experts, 3 slots
    assert c.stats() == before
    st, loads = c.plan([[1, 0]])                     # both still resident
    assert st == 0 and loads == []


def test_repeated_experts_in_one_call_count_once(L):
    c = Cache(L, 8, 2)
    st, loads = c.plan([[3, 5], [5, 3], [3, 5]])
    assert st == 0 and loads == [(3, 0), (5, 1)]
    assert c.stats()[:4] == [1, 2, 0, 2]


def test_reset_empties_the_cache(L):
    c = Cache(L, 8, 4)
    assert c.plan([[1, 2, 3]])[1] == [(1, 0), (2, 1), (3, 2)]
    assert L.lib().seedmm_cache_reset(c.h) == 0
    assert c.stats() == [0, 0, 0, 0, 0]
    assert c.plan([[3, 1]])[1] == [(1, 0), (3, 1)]


def test_empty_call_changes_nothing(L):
    c = Cache(L, 8, 4)
    st, loads = c.plan(np.zeros((0, 2), dtype=np.int32))
    assert st == 0 and loads == []


def test_init_rejects_bad_arguments(L):
    lib = L.lib()
    n = lib.seedmm_cache_state_bytes(8, 4)
    buf = (ctypes.c_uint64 * (n // 8 + 2))()
    base = ctypes.addressof(buf)
    ndev = lib.seedmm_cache_device_bytes(8, 64, 32, 4, 4)
    assert lib.seedmm_cache_state_bytes(8, 9) == 0                   # S > E
    assert lib.seedmm_cache_device_bytes(8, 60, 32, 4, 4) == 0       # H % 8
    assert lib.seedmm_cache_device_bytes(8, 64, 32, 5, 4) == 0       # P
    V = ctypes.c_void_p

    def init(st, sb, dev, db, S=4, pack=FAKE_HOST, eb=FAKE_DEV):
        return lib.seedmm_cache_init(V(st), sb, 8, 64, 32, 4, S, V(pack), V(eb), V(dev), db)

    assert init(base, n - 1, FAKE_DEV, ndev) == L.EINVAL             # state too small
    assert init(base, n, FAKE_DEV, ndev - 1) == L.EINVAL             # device too small
    assert init(base + 4, n, FAKE_DEV, ndev) == L.EALIGN             # state alignment
    assert init(base, n, FAKE_DEV + 16, ndev) == L.EALIGN            # device alignment
    assert init(base, n, FAKE_DEV, ndev, S=0) == L.EINVAL
    assert init(0, n, FAKE_DEV, ndev) == L.EINVAL
    assert init(base, n, FAKE_DEV, ndev, pack=0) == L.EINVAL
    assert init(base, n, FAKE_DEV, ndev, eb=0) == L.EINVAL
    # a handle that was never initialised is rejected
    zero = (ctypes.c_uint64 * (n // 8 + 2))()
    assert lib.seedmm_cache_reset(V(ctypes.addressof(zero))) == L.EINVAL


@pytest.mark.parametrize("H,I,P", [(2048, 1024, 4), (2048, 1024, 3), (64, 32, 4), (24, 16, 3)])
def test_record_layout(L, H, I, P):
    """Nine parts in gate/up/down x seeds/coefs/codes order, each at a multiple of 256
    bytes, none overlapping, each as long as the expert's own stream; the record size is
    a multiple of 256 and the device memory holds S records and the map."""
    lib = L.lib()
    offs = (ctypes.c_size_t * 9)()
    rec = lib.seedmm_cache_record_layout(H, I, P, offs)
    n = I * H // 8
    sizes = [n * 2, (n * P + 3) // 4 * 2, (n + 1) // 2] * 3
    assert rec % 256 == 0
    for i in range(9):
        assert offs[i] % 256 == 0
        end = offs[i] + sizes[i]
        assert end <= (offs[i + 1] if i < 8 else rec)
    assert offs[0] == 0 and rec - (offs[8] + sizes[8]) < 256
    E, S = 10, 3
    assert lib.seedmm_cache_device_bytes(E, H, I, P, S) >= S * rec + 4 * E


def test_cache_moe_rejects_before_planning(L):
    """Argument errors of seedmm_cache_moe return before the plan changes the state and
    before any HIP call (this runs without a GPU)."""
    lib = L.lib()
    c = Cache(L, 8, 2)
    ids = np.array([[1, 2]], dtype=np.int32)
    ip = ids.ctypes.data_as(ctypes.c_void_p)
    F = ctypes.c_void_p(0x30000000)          # 16-byte aligned, never dereferenced
    ws = lib.seedmm_moe_workspace_bytes(1, 2, 8, 64, 32)
    call = lambda ids_p, T, k, x, y, w, wb: lib.seedmm_cache_moe(c.h, ids_p, F, F, T, k, x, y,
                                                                 w, wb, None)
    assert call(ip, -1, 2, F, F, F, ws) == L.EINVAL
    assert call(ip, 1, 0, F, F, F, ws) == L.EINVAL
    assert call(None, 1, 2, F, F, F, ws) == L.EINVAL
    assert call(ip, 1, 2, ctypes.c_void_p(0x30000004), F, F, ws) == L.EALIGN
    assert call(ip, 1, 2, F, F, F, ws - 1) == L.EWORKSPACE
    assert call(ip, 1, 2, F, F, None, ws) == L.EWORKSPACE
    bad = np.array([[1, 8]], dtype=np.int32)
    assert call(bad.ctypes.data_as(ctypes.c_void_p), 1, 2, F, F, F, ws) == L.EINVAL
    many = np.array([[1, 2], [3, 4]], dtype=np.int32)
    ws2 = lib.seedmm_moe_workspace_bytes(2, 2, 8, 64, 32)
    assert call(many.ctypes.data_as(ctypes.c_void_p), 2, 2, F, F, F, ws2) == L.ECAPACITY
    assert c.stats() == [0, 0, 0, 0, 0]
