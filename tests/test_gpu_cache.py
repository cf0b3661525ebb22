"""GPU parity of the expert cache (seedmm_cache_moe): experts resident in pinned host
memory, S device slots, least-recently-used replacement.  The cached layer runs the
same kernels as the resident layer with a slot map, so every call's output must equal
seedmm_moe's on the resident layer bit for bit, across sequences of calls that load
and evict; one call is also checked against the oracle."""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from pseudo_random_weight_amd import seedmm
    return seedmm


def _dev(mat):
    import torch
    return {
        "seeds": torch.from_numpy(mat["seeds"].view(np.int16).copy()).view(torch.uint16).cuda(),
        "coefs": torch.from_numpy(mat["coefs"].view(np.int16).copy()).view(torch.uint16).cuda(),
        "codes": torch.from_numpy(mat["codes"].copy()).cuda(),
        "exp_bias": torch.from_numpy(mat["exp_bias"].copy()).cuda(),
    }


def _layer(E, H, I, P, tag):
    base = synth.config_seed(12)
    return {n: synth.seed_matrix(base, f"{tag}.{n}", *((I, H) if n != "down" else (H, I)), P, E)
            for n in ("gate", "up", "down")}


def _route(tag, T, E, k, hot=None):
    base = synth.config_seed(12)
    ids, w = synth.route_topk(base, tag, T, E, k)
    return ids, w


def _run_sequence(sm, E, H, I, P, S, k, Ts, tag):
    import torch
    host = _layer(E, H, I, P, tag)
    devm = {n: _dev(m) for n, m in host.items()}
    cache = sm.ExpertCache(host, E, H, I, P, S)
    base = synth.config_seed(12)
    for i, T in enumerate(Ts):
        ids, w = _route(f"{tag}.r{i}", T, E, k)
        x = synth.bf16_bits(synth.normal_f32(base, f"{tag}.x{i}", (T, H)))
        xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
        ids_d, w_d = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
        y_ref = sm.moe(ids_d, w_d, xt, E, H, I, P, devm["gate"], devm["up"], devm["down"])
        y = cache.moe(ids, ids_d, w_d, xt)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32)), (i, T)
    return cache.stats(), host


@pytest.mark.parametrize("P", [4, 3])
def test_cache_sequence_matches_the_resident_layer(sm, P):
    """16 experts, 6 slots, top-2: calls of 1..3 tokens (at most 6 distinct experts) load
    and evict on most calls."""
    E, H, I, k, S = 16, 256, 128, 2, 6
    say("cache sequence small", P)
    Ts = [1, 2, 1, 3, 1, 1, 2, 3, 1, 2, 1, 1, 3, 2]
    st, _ = _run_sequence(sm, E, H, I, P, S, k, Ts, f"cs{P}")
    assert st["calls"] == len(Ts)
    assert st["hits"] + st["misses"] == st["uses"]
    assert st["misses"] > st["calls"]          # the sequence does evict


def test_cache_full_size_decode(sm):
    """The 100-expert layer with 33 slots (a third), top-8, one- and four-token calls."""
    E, H, I, P, k, S = 100, 2048, 1024, 4, 8, 33
    say("cache full size")
    st, _ = _run_sequence(sm, E, H, I, P, S, k, [1, 1, 4, 1, 4, 1, 1, 4], "cf")
    assert st["misses"] >= 8


def test_cache_prefill_path(sm):
    """Enough tokens per expert for the prefill kernels, every expert cached."""
    E, H, I, P, k, S = 8, 256, 256, 4, 2, 8
    say("cache prefill")
    _run_sequence(sm, E, H, I, P, S, k, [600, 600], "cp")


def test_cache_matches_the_oracle(sm, oracle):
    import torch
    E, H, I, P, k, S, T = 12, 256, 128, 4, 3, 4, 1
    say("cache vs oracle")
    host = _layer(E, H, I, P, "co")
    cache = sm.ExpertCache(host, E, H, I, P, S)
    base = synth.config_seed(12)
    for i in range(4):
        ids, w = _route(f"co.r{i}", T, E, k)
        x = synth.bf16_bits(synth.normal_f32(base, f"co.x{i}", (T, H)))
        xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
        y = cache.moe(ids, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), xt)
        torch.cuda.synchronize()
        ref = oracle.moe(ids, w, synth.bf16_bits_to_f32(x), E, H, I, P,
                         host["gate"], host["up"], host["down"])
        y = y.cpu().numpy()
        err = np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref)
        assert err <= 1e-2, (i, err)


def test_cache_capacity_error_leaves_the_cache_usable(sm):
    import torch
    E, H, I, P, k, S = 8, 256, 128, 4, 2, 2
    say("cache capacity")
    host = _layer(E, H, I, P, "cc")
    devm = {n: _dev(m) for n, m in host.items()}
    cache = sm.ExpertCache(host, E, H, I, P, S)
    ids = np.array([[0, 1], [2, 3]], dtype=np.int32)
    w = np.full((2, 2), 0.5, dtype=np.float32)
    x = torch.randn(2, H).to(torch.bfloat16).cuda()
    with pytest.raises(sm.SeedmmError) as ei:
        cache.moe(ids, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), x)
    assert ei.value.status == sm.ECAPACITY
    one = ids[:1].copy()
    y = cache.moe(one, torch.from_numpy(one).cuda(), torch.from_numpy(w[:1]).cuda(), x[:1])
    y_ref = sm.moe(torch.from_numpy(one).cuda(), torch.from_numpy(w[:1]).cuda(), x[:1].contiguous(),
                   E, H, I, P, devm["gate"], devm["up"], devm["down"])
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y_ref.cpu().numpy())


def test_cache_refuses_short_buffers_before_the_plan(sm):
    """The binding checks y, x and topk_w against T before the call plans (and so
    changes) the cache state."""
    import torch
    E, H, I, P, k, S = 8, 256, 128, 4, 2, 4
    say("cache short buffers")
    host = _layer(E, H, I, P, "csb")
    cache = sm.ExpertCache(host, E, H, I, P, S)
    ids = np.array([[0, 1], [2, 3]], dtype=np.int32)
    ids_d = torch.from_numpy(ids).cuda()
    w = torch.full((2, 2), 0.5, dtype=torch.float32, device="cuda")
    x = torch.randn(2, H).to(torch.bfloat16).cuda()
    with pytest.raises(ValueError):
        cache.moe(ids, ids_d, w, x, y=torch.empty((1, H), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        cache.moe(ids, ids_d, w, x[:1].contiguous())
    with pytest.raises(ValueError):
        cache.moe(ids, ids_d, w[:1].contiguous(), x)
    assert cache.stats()["calls"] == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("P", [4, 3])
def test_cache_per_expert_biases_and_degenerate_blocks(sm, oracle, P):
    """Every expert's gate, up and down with an exp_bias of its own (gate outputs of order
    1, where silu is curved) and planted seed-0 and zero-coefficient blocks: the cached
    layer reads each expert's biases by expert id, not by slot, so its output equals the
    resident layer's bit for bit across loads and evictions, and the oracle's within
    1e-2 (a slot-indexed bias would scale whole experts by powers of two)."""
    import torch
    E, H, I, k, S = 12, 256, 128, 2, 4   # a 2-token call touches up to 4 experts
    say("cache per-expert biases", P)
    base = synth.config_seed(26)
    host = {}
    for n, lo, hi in (("gate", -22, -20), ("up", -22, -18), ("down", -21, -17)):
        M, K = (I, H) if n != "down" else (H, I)
        eb = synth.uniform_ints(base, f"cb{P}.{n}.eb", E, lo, hi)
        m = synth.seed_matrix(base, f"cb{P}.{n}", M, K, P, E, exp_bias=eb)
        m = synth.plant_degenerate(m, P, base, f"cb{P}.{n}.deg", frac=0.03)
        host[n] = {key: m[key] for key in ("seeds", "coefs", "codes", "exp_bias")}
    assert len(set(host["gate"]["exp_bias"].tolist())) > 1
    devm = {n: _dev(m) for n, m in host.items()}
    cache = sm.ExpertCache(host, E, H, I, P, S)
    for i, T in enumerate([1, 1, 2, 1, 1, 2, 1]):
        ids, w = _route(f"cb{P}.r{i}", T, E, k)
        x = synth.bf16_bits(synth.normal_f32(base, f"cb{P}.x{i}", (T, H)))
        xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
        ids_d, w_d = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
        y = cache.moe(ids, ids_d, w_d, xt)
        y_ref = sm.moe(ids_d, w_d, xt, E, H, I, P, devm["gate"], devm["up"], devm["down"])
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        assert np.array_equal(y.view(np.uint32), y_ref.cpu().numpy().view(np.uint32)), (i, T)
        ref = oracle.moe(ids, w, synth.bf16_bits_to_f32(x), E, H, I, P,
                         host["gate"], host["up"], host["down"])
        err = np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref)
        assert err <= 1e-2, (i, err)
    assert cache.stats()["misses"] > S
