"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Weights are compared bit for bit; products by relative L2 error
||y - y_ref|| / ||y_ref|| (fp32 activations: 1e-5; bf16 activations with fp32
accumulation: 1e-2).  Full-size workloads are checked on sampled outputs the oracle
computes one token at a time.
"""
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


def dev(mat):
    import torch
    return {
        "seeds": torch.from_numpy(mat["seeds"].view(np.int16).copy()).view(torch.uint16).cuda(),
        "coefs": torch.from_numpy(mat["coefs"].view(np.int16).copy()).view(torch.uint16).cuda(),
        "codes": torch.from_numpy(mat["codes"].copy()).cuda(),
        "exp_bias": torch.from_numpy(mat["exp_bias"].copy()).cuda(),
        "exp_bias_host": mat["exp_bias"].copy(),
    }


def rel_l2(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def bf16_tensor(xf32):
    import torch
    bits = synth.bf16_bits(xf32)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda(), \
        synth.bf16_bits_to_f32(bits)


SHAPES = [
    (256, 512),      # the small parity workload (vector path)
    (37, 104),       # ragged rows, K not a multiple of 64 (per-block path)
    (48, 8),         # a single block per row
    (130, 2048),     # many segments, ragged row tile
    (64, 576),       # K % 64 == 0 but not a multiple of the 4-quarter stride
]


@pytest.mark.parametrize("P", [4, 3])
@pytest.mark.parametrize("M,K", SHAPES)
def test_reconstruct_is_bit_exact(sm, oracle, P, M, K):
    import torch
    say("reconstruct", M, K, P)
    mat = synth.seed_matrix(synth.config_seed(0), f"rc{M}x{K}", M, K, P)
    d = dev(mat)
    W = sm.reconstruct(d, M, K, P, torch.float32)
    Wb = sm.reconstruct(d, M, K, P, torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.reconstruct_f32(mat, M, K, P)
    refb = oracle.reconstruct_bf16(mat, M, K, P)
    np.testing.assert_array_equal(W.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    np.testing.assert_array_equal(Wb.cpu().view(torch.int16).numpy().view(np.uint16), refb)


def test_reconstruct_extreme_exponents(sm, oracle):
    import torch
    say("reconstruct exponents")
    M, K, P = 16, 256, 4
    for eb in (-100, -4, 0, 37, 100):
        mat = synth.seed_matrix(synth.config_seed(0), f"eb{eb}", M, K, P, exp_bias=eb)
        W = sm.reconstruct(dev(mat), M, K, P, torch.float32)
        torch.cuda.synchronize()
        ref = oracle.reconstruct_f32(mat, M, K, P)
        np.testing.assert_array_equal(W.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("P", [4, 3])
@pytest.mark.parametrize("M,K", SHAPES)
def test_gemv_fp32_matches_oracle(sm, oracle, P, M, K):
    import torch
    say("gemv fp32", M, K, P)
    base = synth.config_seed(0)
    mat = synth.seed_matrix(base, f"gv{M}x{K}", M, K, P)
    x = synth.normal_f32(base, f"x{K}", (K,))
    y = sm.gemv(dev(mat), torch.from_numpy(x).cuda(), M, K, P)
    torch.cuda.synchronize()
    ref = oracle.gemv(mat, x[None], M, K, P)[0]
    assert rel_l2(y.cpu().numpy(), ref) <= 1e-5


def test_gemv_one_hot_is_bit_exact(sm, oracle):
    import torch
    say("gemv one-hot")
    M, K, P = 256, 512, 4
    mat = synth.seed_matrix(synth.config_seed(0), "onehot", M, K, P)
    d = dev(mat)
    Wref = oracle.reconstruct_f32(mat, M, K, P)
    for k in (0, 5, 8, 263, 511):
        x = torch.zeros(K, dtype=torch.float32, device="cuda")
        x[k] = 1.0
        y = sm.gemv(d, x, M, K, P)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), Wref[:, k])


def test_gemv_under_another_stream_waits_for_its_inputs(sm, oracle):
    """seedmm_gemv runs on the null stream: under another current stream the binding orders
    it after that stream's pending work.  x is written on the side stream behind a bounded
    spin, and y is read back on that stream."""
    import torch
    say("gemv under a side stream")
    M, K, P = 256, 512, 4
    base = synth.config_seed(0)
    mat = synth.seed_matrix(base, "gvside", M, K, P)
    d = dev(mat)
    x_host = synth.normal_f32(base, "xside", (K,))
    src = torch.from_numpy(x_host).cuda()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        x = torch.zeros(K, dtype=torch.float32, device="cuda")
        torch.cuda._sleep(2_000_000)           # a bounded spin that holds the stream back
        x.copy_(src)
        y = sm.gemv(d, x, M, K, P)
        y2 = y * 1.0
    side.synchronize()
    ref = oracle.gemv(mat, x_host[None], M, K, P)[0]
    assert rel_l2(y2.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("N", [2, 3, 5, 9])
def test_gemv_ex_fp32_batches(sm, oracle, N):
    import torch
    say("gemv_ex fp32", N)
    M, K, P = 96, 1024, 4
    base = synth.config_seed(0)
    mat = synth.seed_matrix(base, "gvb", M, K, P)
    x = synth.normal_f32(base, f"xb{N}", (N, K))
    y = sm.gemv_ex(dev(mat), torch.from_numpy(x).cuda(), M, K, P)
    torch.cuda.synchronize()
    ref = oracle.gemv(mat, x, M, K, P)
    assert rel_l2(y.cpu().numpy(), ref) <= 1e-5
    # linearity: W (a + b) = W a + W b up to rounding
    y2 = sm.gemv_ex(dev(mat), torch.from_numpy(2 * x).cuda(), M, K, P)
    torch.cuda.synchronize()
    assert rel_l2(y2.cpu().numpy(), 2 * ref) <= 1e-5


def test_gemv_ex_fp32_rows_beyond_one_launch(sm, oracle):
    """fp32 products take 4 rows of X per workgroup row, and a launch holds at most 65,535
    workgroup rows: N = 4 * 65535 + 5 runs as two launches.  Every row within 1e-5 of the
    oracle, and the rows of the second launch bit-equal to the same rows in a call of
    their own (a row's sums do not depend on the other rows)."""
    import torch
    M, K, P, N = 16, 64, 4, 4 * 65535 + 5
    say("gemv_ex fp32 rows beyond one launch", N)
    base = synth.config_seed(0)
    mat = synth.seed_matrix(base, "gvbig", M, K, P)
    x = synth.normal_f32(base, "xbig", (N, K))
    d = dev(mat)
    xt = torch.from_numpy(x).cuda()
    y = sm.gemv_ex(d, xt, M, K, P)
    tail = sm.gemv_ex(d, xt[N - 9:].contiguous(), M, K, P)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle.gemv(mat, x, M, K, P)
    err = np.linalg.norm(y.astype(np.float64) - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert err.max() <= 1e-5, int(err.argmax())
    np.testing.assert_array_equal(y[N - 9:].view(np.uint32), tail.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("P", [4, 3])
@pytest.mark.parametrize("N", [1, 8, 16, 17, 64, 65, 300])
def test_gemv_ex_bf16_matches_oracle(sm, oracle, P, N):
    import torch
    say("gemv_ex bf16", N, P)
    M, K = 160, 768
    base = synth.config_seed(1)
    mat = synth.seed_matrix(base, f"gx{P}", M, K, P)
    xt, x32 = bf16_tensor(synth.normal_f32(base, f"xx{N}", (N, K)))
    y = sm.gemv_ex(dev(mat), xt, M, K, P)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle.gemv(mat, x32, M, K, P)
    assert rel_l2(y, ref) <= 1e-2
    # the kernel multiplies the bf16 (nearest-even) weights exactly with fp32 sums
    Wb = synth.bf16_bits_to_f32(oracle.reconstruct_bf16(mat, M, K, P)).astype(np.float64)
    ref_b = x32.astype(np.float64) @ Wb.T
    assert rel_l2(y, ref_b) <= 1e-5


@pytest.mark.parametrize("P", [4, 3])
@pytest.mark.parametrize("M,K", SHAPES + [(40, 1032), (24, 2056)])
def test_gemv_ex_bf16_shapes(sm, oracle, P, M, K):
    """bf16 products over ragged shapes: the per-block path with several K iterations
    per wave (K % 64 != 0 and more than 16 segments) and the vector path's tails."""
    import torch
    say("gemv_ex bf16 shape", M, K, P)
    base = synth.config_seed(1)
    mat = synth.seed_matrix(base, f"gs{P}.{M}.{K}", M, K, P)
    xt, x32 = bf16_tensor(synth.normal_f32(base, f"xs{M}.{K}", (5, K)))
    y = sm.gemv_ex(dev(mat), xt, M, K, P)
    torch.cuda.synchronize()
    Wb = synth.bf16_bits_to_f32(oracle.reconstruct_bf16(mat, M, K, P)).astype(np.float64)
    ref_b = x32.astype(np.float64) @ Wb.T
    assert rel_l2(y.cpu().numpy(), ref_b) <= 1e-5
    assert rel_l2(y.cpu().numpy(), oracle.gemv(mat, x32, M, K, P)) <= 1e-2


def test_dispatch_groups_pairs_in_order(sm):
    import torch
    for (T, E, k) in [(1, 100, 8), (64, 100, 8), (37, 5, 3), (4096, 100, 8), (3, 16, 1),
                      (1500, 10, 7)]:
        say("dispatch", T, E, k)
        ids, _ = synth.route_topk(synth.config_seed(2), f"d{T}", T, E, k)
        counts, lists = sm.moe_dispatch(torch.from_numpy(ids).cuda(), E)
        torch.cuda.synchronize()
        counts = counts.cpu().numpy()
        lists = lists.cpu().numpy()
        flat = ids.reshape(-1)
        np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
        for e in range(E):
            np.testing.assert_array_equal(lists[e, :counts[e]], np.nonzero(flat == e)[0])


def test_layer_dispatch_many_pairs_in_order(sm):
    """The layer's own dispatch for many pairs (two launches over expert x tile
    workgroups): the per-expert lists it leaves at the start of its workspace (counts,
    then the lists from the next 256-byte boundary) hold each expert's pairs in pair
    order."""
    import torch
    E, H, I, P, k = 100, 2048, 1024, 4, 8
    for T in (1500, 4096):                      # 12,000 and 32,768 pairs: 2 and 4 tiles
        say("layer dispatch", T)
        gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 2, f"ld{T}")
        g, u, d = dev(gate), dev(up), dev(down)
        xt, _ = bf16_tensor(x)
        ws = torch.empty(sm.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
        sm.moe(torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), xt, E, H, I, P, g, u, d,
               workspace=ws)
        torch.cuda.synchronize()
        raw = ws.cpu().numpy()
        counts = raw[:4 * E].view(np.int32)
        off = (4 * E + 255) // 256 * 256
        lists = raw[off:off + 4 * E * T].view(np.int32).reshape(E, T)
        flat = ids.reshape(-1)
        np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
        for e in range(E):
            np.testing.assert_array_equal(lists[e, :counts[e]], np.nonzero(flat == e)[0])


_LAYERS = {}


def layer(E, H, I, P, cfg):
    """Seed-coded gate/up/down stacks of one layer (cached: the 100-expert layer is large)."""
    key = (E, H, I, P, cfg)
    if key not in _LAYERS:
        base = synth.config_seed(cfg)
        _LAYERS[key] = (synth.seed_matrix(base, "gate", I, H, P, E),
                        synth.seed_matrix(base, "up", I, H, P, E),
                        synth.seed_matrix(base, "down", H, I, P, E))
    return _LAYERS[key]


def moe_case(T, E, H, I, P, k, cfg, tag):
    base = synth.config_seed(cfg)
    gate, up, down = layer(E, H, I, P, cfg)
    ids, w = synth.route_topk(base, tag + ".router", T, E, k)
    x = synth.normal_f32(base, tag + ".x", (T, H))
    return gate, up, down, ids, w, x


def run_moe(sm, gate, up, down, ids, w, x, E, H, I, P):
    import torch
    xt, x32 = bf16_tensor(x)
    y = sm.moe(torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), xt, E, H, I, P,
               dev(gate), dev(up), dev(down))
    torch.cuda.synchronize()
    return y.cpu().numpy(), x32


@pytest.mark.parametrize("T", [1, 8])
def test_single_expert_ffn(sm, oracle, T):
    # one SwiGLU expert, hidden 2048, intermediate 768, P=4 (top-1 routing, weight 1)
    say("expert ffn", T)
    E, H, I, P = 1, 2048, 768, 4
    gate, up, down, _, _, x = moe_case(T, E, H, I, P, 1, 1, "ffn")
    ids = np.zeros((T, 1), dtype=np.int32)
    w = np.ones((T, 1), dtype=np.float32)
    y, x32 = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    ref = oracle.expert(gate, up, down, x32, H, I, P)
    assert rel_l2(y, ref) <= 1e-2


@pytest.mark.parametrize("P,T", [(4, 1), (4, 4), (3, 1)])
def test_moe_layer_full(sm, oracle, P, T):
    # the 100-expert layer, 2048 -> 1024 -> 2048, top-8, every output checked
    say("moe full", P, T)
    E, H, I, k = 100, 2048, 1024, 8
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 2 if P == 4 else 3, f"moe{P}")
    y, x32 = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    ref = oracle.moe(ids, w, x32, E, H, I, P, gate, up, down)
    assert rel_l2(y, ref) <= 1e-2


@pytest.mark.parametrize("P,T", [(4, 16), (4, 64), (3, 16), (4, 160)])
def test_moe_layer_sampled_tokens(sm, oracle, P, T):
    say("moe sampled", P, T)
    E, H, I, k = 100, 2048, 1024, 8
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 2 if P == 4 else 3, f"moeS{P}")
    y, x32 = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    for t in (0, T // 2, T - 1):
        ref = oracle.moe(ids[t:t + 1], w[t:t + 1], x32[t:t + 1], E, H, I, P, gate, up, down)
        assert rel_l2(y[t], ref[0]) <= 1e-2, t


def test_moe_output_independent_of_batch(sm):
    """A token's output bits do not depend on the other tokens of its batch (128 vs 129
    tokens: different tile fill and expert lists)."""
    E, H, I, P, k = 100, 2048, 1024, 4, 8
    say("moe batch independence 128 vs 129 tokens")
    gate, up, down, ids, w, x = moe_case(129, E, H, I, P, k, 2, "paths")
    y_big, _ = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)        # 1032 pairs
    y_small, _ = run_moe(sm, gate, up, down, ids[:128], w[:128], x[:128], E, H, I, P)
    assert np.array_equal(y_small.view(np.uint32), y_big[:128].view(np.uint32))
    # one token takes the dispatch-free path (its top_k slots name the experts)
    for t in (0, 77):
        y_one, _ = run_moe(sm, gate, up, down, ids[t:t + 1], w[t:t + 1], x[t:t + 1], E, H, I, P)
        assert np.array_equal(y_one.view(np.uint32), y_big[t:t + 1].view(np.uint32)), t


@pytest.mark.parametrize("E,H,I,P,k", [
    (6, 200, 136, 4, 2),      # K % 64 != 0: the per-block stream path
    (12, 2048, 1024, 3, 4),   # P = 3, vector path
    (4, 16640, 64, 4, 2),     # gate/up K above the one-token kernel's LDS row limit
])
def test_one_token_matches_its_batch_and_the_oracle(sm, oracle, E, H, I, P, k):
    """One token runs the one-token kernels (activation row in LDS) unless K is too long
    for them; either way its output equals the same token's inside a 3-token batch bit
    for bit, and the oracle within tolerance."""
    say("one token", E, H, I, P, k)
    gate, up, down, ids, w, x = moe_case(3, E, H, I, P, k, 4, f"one{H}x{I}")
    y3, x32 = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    for t in range(3):
        y1, _ = run_moe(sm, gate, up, down, ids[t:t + 1], w[t:t + 1], x[t:t + 1], E, H, I, P)
        assert np.array_equal(y1.view(np.uint32), y3[t:t + 1].view(np.uint32)), t
        ref = oracle.moe(ids[t:t + 1], w[t:t + 1], x32[t:t + 1], E, H, I, P, gate, up, down)
        assert rel_l2(y1[0], ref[0]) <= 1e-2, t


@pytest.mark.parametrize("E,H,I,P,k", [
    (10, 256, 192, 4, 2),     # two slots: one wave pair of the workgroup
    (10, 192, 128, 4, 3),     # odd top_k: the fourth slot's lanes have no expert
    (12, 128, 256, 3, 5),     # P = 3
    (16, 320, 64, 4, 7),
    (16, 64, 4160, 4, 8),     # top_k * I * 2 B above 64 KB: per-slot outputs + combine
    (16, 256, 128, 4, 12),    # top_k above 8: per-slot outputs + the general combine
])
def test_one_token_down_adds_the_slots(sm, oracle, E, H, I, P, k):
    """One token with one P: the down kernel adds the top_k slot outputs itself in slot
    order (for top_k <= 8 when top_k * I bf16 fit its 64 KB LDS budget; otherwise the
    per-slot outputs and the combine run).  Either way each token's bits equal those it gets inside a batch
    (dispatch, decode kernels, combine), and the batch matches the oracle."""
    say("one-token down with the slot sum", E, H, I, P, k)
    gate, up, down, ids, w, x = moe_case(3, E, H, I, P, k, 6, f"d1s{k}")
    y_b, x32 = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    for t in range(3):
        y1, _ = run_moe(sm, gate, up, down, ids[t:t + 1], w[t:t + 1], x[t:t + 1], E, H, I, P)
        assert np.array_equal(y1[0].view(np.uint32), y_b[t].view(np.uint32)), t
    ref = oracle.moe(ids, w, x32, E, H, I, P, gate, up, down)
    assert rel_l2(y_b, ref) <= 1e-2


@pytest.mark.parametrize("T", [1, 4])
def test_moe_graph_replays_match_eager(sm, T):
    """The layer call captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, gives the eager result bit for bit.  The workspace
    is filled with 0xFF before each replay, so no replay may depend on its contents
    (one token: the dispatch-free path; four tokens: the dispatch lists)."""
    import torch
    E, H, I, P, k = 100, 2048, 1024, 4, 8
    say("moe graph replay", T)
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 2, "graph")
    y_ref, _ = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    g, u, d = dev(gate), dev(up), dev(down)
    ids_t, w_t = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    xt, _ = bf16_tensor(x)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(sm.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sm.moe(ids_t, w_t, xt, E, H, I, P, g, u, d, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    G = torch.cuda.CUDAGraph()
    with torch.cuda.graph(G):
        sm.moe(ids_t, w_t, xt, E, H, I, P, g, u, d, y=y, workspace=ws)
    other = torch.from_numpy(np.roll(ids, 1, axis=0)).cuda()
    for rep in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xFF)
        G.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), rep
        # eager work between replays, on the same workspace
        sm.moe(other, w_t, xt, E, H, I, P, g, u, d, y=torch.empty_like(y), workspace=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("P", [4, 3])
def test_moe_prefill_path_small(sm, oracle, P):
    # >= 64 tokens per expert selects the prefill shape; small dims keep the oracle quick
    say("moe prefill small", P)
    T, E, H, I, k = 600, 8, 256, 128, 2
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 4, "pfs" if P == 4 else "pfs3")
    y, x32 = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    ref = oracle.moe(ids, w, x32, E, H, I, P, gate, up, down)
    assert rel_l2(y, ref) <= 1e-2


def _slot_sum(ws, T, k, E, H, I):
    """y as the combine defines it from the per-slot outputs o (fp32 [T*k][H]) left in the
    layer's workspace: o[t*k] + o[t*k+1] + ... in slot order, in fp32."""
    al = lambda v: (v + 255) // 256 * 256
    off = al(4 * E) + al(4 * E * T) + al(2 * T * k * I)
    o = ws[off:off + 4 * T * k * H].cpu().numpy().view(np.float32).reshape(T, k, H)
    y = o[:, 0].copy()
    for s in range(1, k):
        y = y + o[:, s]
    return y


def _raw_events(n):
    """n raw hipEvent_t handles (ints) from the HIP runtime, for the timed layer call."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    out = []
    for _ in range(n):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        out.append(h.value)
    return out


@pytest.mark.parametrize("E,P,T", [(8, 4, 600), (7, 3, 600), (12, 4, 16), (5, 3, 9), (8, 4, 1),
                                   (7, 3, 1)])
def test_moe_prefill_two_streams(sm, oracle, E, P, T):
    """A layer call over several tokens with one P and a caller's side stream
    (seedmm_moe_ex) runs each half of the experts on its own stream, for the prefill
    kernels (T = 600 here) and the decode ones (T = 16, 9); a single token runs on one
    stream even when a side stream is given (T = 1).  Its output equals the single-stream
    order of the timed call bit for bit (every expert served exactly once, whatever the
    split point), matches the oracle, and graph replays of it reproduce the eager result
    bit for bit."""
    import torch
    H, I, k = 256, 256, 2
    say("moe two streams", E, P, T)
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 5, f"pf2s{E}")
    g, u, d = dev(gate), dev(up), dev(down)
    ids_t, w_t = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    xt, x32 = bf16_tensor(x)
    ws = torch.empty(sm.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    side = sm.SideStream()
    y_two = sm.moe(ids_t, w_t, xt, E, H, I, P, g, u, d, workspace=ws, side=side)
    torch.cuda.synchronize()
    y_one = sm.moe(ids_t, w_t, xt, E, H, I, P, g, u, d, events=_raw_events(5))
    torch.cuda.synchronize()
    y_two, y_one = y_two.cpu().numpy(), y_one.cpu().numpy()
    assert np.array_equal(y_two.view(np.uint32), y_one.view(np.uint32))
    if T > 1:
        # y is the slot-ordered sum of the per-slot outputs (ws still holds the two-stream
        # call's: the timed call had its own workspace)
        assert np.array_equal(y_two.view(np.uint32), _slot_sum(ws, T, k, E, H, I).view(np.uint32))
    else:
        # one token: its down kernel adds the slots itself (no per-slot outputs in the
        # workspace); the same token twice in a batch (dispatch, decode kernels, combine)
        # gives the same bits
        x2 = np.repeat(x, 2, axis=0)
        xt2, _ = bf16_tensor(x2)
        y_b = sm.moe(torch.from_numpy(np.repeat(ids, 2, axis=0)).cuda(),
                     torch.from_numpy(np.repeat(w, 2, axis=0)).cuda(), xt2, E, H, I, P, g, u, d)
        torch.cuda.synchronize()
        y_b = y_b.cpu().numpy()
        for t in range(2):
            assert np.array_equal(y_b[t].view(np.uint32), y_two[0].view(np.uint32)), t
    ref = oracle.moe(ids, w, x32, E, H, I, P, gate, up, down)
    assert rel_l2(y_two, ref) <= 1e-2
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    G = torch.cuda.CUDAGraph()
    with torch.cuda.graph(G):
        sm.moe(ids_t, w_t, xt, E, H, I, P, g, u, d, y=y, workspace=ws, side=side)
    other = torch.from_numpy(np.roll(ids, 1, axis=0)).cuda()
    for rep in range(3):
        y.fill_(float("nan"))
        ws.fill_(0xFF)
        G.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_two.view(np.uint32)), rep
        # eager work between replays, on the same workspace and side stream
        sm.moe(other, w_t, xt, E, H, I, P, g, u, d, y=torch.empty_like(y), workspace=ws,
               side=side)
        torch.cuda.synchronize()
    # without a side stream (seedmm_moe): the same bits
    y_plain = sm.moe(ids_t, w_t, xt, E, H, I, P, g, u, d)
    torch.cuda.synchronize()
    assert np.array_equal(y_plain.cpu().numpy().view(np.uint32), y_two.view(np.uint32))


def test_moe_on_a_non_current_stream(sm):
    """A layer call on a stream other than torch's current one, with the output and the
    workspace allocated by the binding (on that stream) and a side stream: the result
    equals the call on the current stream bit for bit, also when the allocator reuses
    freed blocks between calls."""
    import torch
    E, H, I, P, k, T = 12, 256, 256, 4, 2, 40
    say("moe non-current stream")
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 5, "ncs")
    g, u, d = dev(gate), dev(up), dev(down)
    ids_t, w_t = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    xt, _ = bf16_tensor(x)
    y_ref = sm.moe(ids_t, w_t, xt, E, H, I, P, g, u, d).cpu().numpy()
    s = torch.cuda.Stream()
    side = sm.SideStream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        y = sm.moe(ids_t, w_t, xt, E, H, I, P, g, u, d, stream=s, side=side if rep else None)
        outs.append(y)
        junk = torch.full((1 << 20,), rep, dtype=torch.float32, device="cuda")   # allocator churn
        del junk
    s.synchronize()
    for y in outs:
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


def test_moe_prefill_full_size_sampled(sm, oracle):
    # 4096 tokens through the 100-expert top-8 layer; sampled tokens vs the oracle
    say("moe prefill 4096")
    import torch
    T, E, H, I, P, k = 4096, 100, 2048, 1024, 4, 8
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 4, "pf")
    xt, x32 = bf16_tensor(x)
    ws = torch.empty(sm.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    y = sm.moe(torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), xt, E, H, I, P,
               dev(gate), dev(up), dev(down), workspace=ws)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.all(np.isfinite(y))
    # the combine adds every token's slot rows in slot order, bit for bit
    assert np.array_equal(y.view(np.uint32), _slot_sum(ws, T, k, E, H, I).view(np.uint32))
    for t in (0, 1234, T - 1):
        ref = oracle.moe(ids[t:t + 1], w[t:t + 1], x32[t:t + 1], E, H, I, P, gate, up, down)
        assert rel_l2(y[t], ref[0]) <= 1e-2, t


def test_moe_edge_cases(sm, oracle):
    import torch
    E, H, I, P = 6, 192, 96, 4        # H, I not multiples of 64: per-block path
    gate, up, down, ids, w, x = moe_case(40, E, H, I, P, 2, 5, "edge")
    say("moe all tokens to one expert")
    ids1 = np.full((40, 1), 3, dtype=np.int32)
    w1 = np.ones((40, 1), dtype=np.float32)
    y, x32 = run_moe(sm, gate, up, down, ids1, w1, x, E, H, I, P)
    ref = oracle.moe(ids1, w1, x32, E, H, I, P, gate, up, down)
    assert rel_l2(y, ref) <= 1e-2
    say("moe ragged dims, several experts empty")
    y, x32 = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    ref = oracle.moe(ids, w, x32, E, H, I, P, gate, up, down)
    assert rel_l2(y, ref) <= 1e-2
    say("moe empty batch")
    yt = sm.moe(torch.zeros((0, 2), dtype=torch.int32, device="cuda"),
                torch.zeros((0, 2), dtype=torch.float32, device="cuda"),
                torch.zeros((0, H), dtype=torch.bfloat16, device="cuda"), E, H, I, P,
                dev(gate), dev(up), dev(down))
    assert yt.shape == (0, H)


@pytest.mark.parametrize("P", [4, 3])
def test_moe_per_block_path_long_rows(sm, oracle, P):
    """H, I not multiples of 64 and long enough that every wave loops over several K
    segments (per-block stream loads with the next segment prefetched)."""
    E, H, I, T, k = 4, 1032, 264, 6, 2
    say("moe per-block long rows", P)
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 7, f"long{P}")
    y, x32 = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    ref = oracle.moe(ids, w, x32, E, H, I, P, gate, up, down)
    assert rel_l2(y, ref) <= 1e-2


def test_moe_is_deterministic_and_permutation_equivariant(sm):
    say("moe determinism")
    E, H, I, P, k, T = 100, 2048, 1024, 4, 8, 16
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 2, "det")
    y1, _ = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    y2, _ = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    np.testing.assert_array_equal(y1, y2)
    perm = np.random.default_rng(0).permutation(T)
    y3, _ = run_moe(sm, gate, up, down, ids[perm], w[perm], x[perm], E, H, I, P)
    np.testing.assert_array_equal(y3, y1[perm])


# ---------------------------------------------------------------------------------
# Encoder: the exhaustive seed search on the GPU against the oracle's search
# ---------------------------------------------------------------------------------
def _search_case(M, K, tag, scale=0.02):
    base = synth.config_seed(7)
    return (synth.normal_f32(base, tag + ".W", (M, K)) * scale).astype(np.float32)


@pytest.mark.parametrize("P", [4, 3])
@pytest.mark.parametrize("weighted", [False, True])
def test_search_matches_oracle_bit_for_bit(sm, oracle, P, weighted):
    """Seeds, coefficient and code streams and every block's squared error equal the
    oracle's search exactly (11 blocks: a ragged group of four, P = 3 words shared
    across blocks)."""
    import torch
    M, K = 1, 88
    say("search vs oracle", P, weighted)
    W = _search_case(M, K, f"s{P}{weighted}")
    colw = None
    if weighted:
        colw = np.abs(synth.normal_f32(synth.config_seed(7), f"cw{P}", (K,))).astype(np.float32) + 0.1
    ref = oracle.search_matrix(W, P, -4, colw)
    got = sm.search(torch.from_numpy(W).cuda(), P, -4,
                    None if colw is None else torch.from_numpy(colw).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got["seeds"].cpu().view(torch.int16).numpy().view(np.uint16), ref["seeds"])
    np.testing.assert_array_equal(got["coefs"].cpu().view(torch.int16).numpy().view(np.uint16), ref["coefs"])
    np.testing.assert_array_equal(got["codes"].cpu().numpy(), ref["codes"])
    np.testing.assert_array_equal(got["err"].cpu().numpy().view(np.uint64), ref["err"].view(np.uint64))


@pytest.mark.parametrize("P,weighted", [(4, False), (3, False), (4, True)])
def test_search_edge_blocks_match_oracle(sm, oracle, P, weighted):
    """Blocks at the edges of the seed bound, against the oracle bit for bit: all zero
    (nothing to bound), constant, too small for any nonzero coefficient, large enough
    to clamp, exact seed-coded blocks (best error 0), a single nonzero weight, and with
    importance weights, columns of weight 0."""
    import torch
    say("search edge blocks", P, weighted)
    base = synth.config_seed(9)
    planted = oracle.reconstruct_f32(synth.seed_matrix(base, f"edge{P}", 1, 16, P), 1, 16, P)[0]
    rnd = synth.normal_f32(base, "edge.r", (8,))
    blocks = [
        np.zeros(8, np.float32),
        np.full(8, 0.01, np.float32),
        np.full(8, -3.0e-3, np.float32),
        (rnd * 1e-12).astype(np.float32),
        (rnd * 50.0).astype(np.float32),
        planted[:8], planted[8:],
        np.array([0, 0, 0, 0.02, 0, 0, 0, 0], np.float32),
        (rnd * 0.02).astype(np.float32),
    ]
    W = np.concatenate(blocks)[None, :]                 # one row of 9 blocks (ragged group)
    K = W.shape[1]
    colw = None
    if weighted:
        colw = np.abs(synth.normal_f32(base, "edge.cw", (K,))).astype(np.float32) + 0.1
        colw[::3] = 0.0                                  # some columns carry no weight
    ref = oracle.search_matrix(W, P, -4, colw)
    got = sm.search(torch.from_numpy(W).cuda(), P, -4,
                    None if colw is None else torch.from_numpy(colw).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got["seeds"].cpu().view(torch.int16).numpy().view(np.uint16), ref["seeds"])
    np.testing.assert_array_equal(got["coefs"].cpu().view(torch.int16).numpy().view(np.uint16), ref["coefs"])
    np.testing.assert_array_equal(got["codes"].cpu().numpy(), ref["codes"])
    np.testing.assert_array_equal(got["err"].cpu().numpy().view(np.uint64), ref["err"].view(np.uint64))


@pytest.mark.parametrize("P,weighted,M", [(4, False, 4), (3, True, 2)])
def test_search_many_blocks_match_oracle(sm, oracle, P, weighted, M):
    """Many random blocks (256 or 128), so the seed bound prunes in every state of the
    running best: the whole encoding equals the oracle's bit for bit."""
    import torch
    K = 512
    say("search many blocks", P, weighted, M * K // 8)
    W = _search_case(M, K, f"many{P}{weighted}")
    colw = None
    if weighted:
        colw = np.abs(synth.normal_f32(synth.config_seed(7), f"cwm{P}", (K,))).astype(np.float32) + 0.1
    ref = oracle.search_matrix(W, P, -4, colw)
    got = sm.search(torch.from_numpy(W).cuda(), P, -4,
                    None if colw is None else torch.from_numpy(colw).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got["seeds"].cpu().view(torch.int16).numpy().view(np.uint16), ref["seeds"])
    np.testing.assert_array_equal(got["coefs"].cpu().view(torch.int16).numpy().view(np.uint16), ref["coefs"])
    np.testing.assert_array_equal(got["codes"].cpu().numpy(), ref["codes"])
    np.testing.assert_array_equal(got["err"].cpu().numpy().view(np.uint64), ref["err"].view(np.uint64))


@pytest.mark.parametrize("P", [4, 3])
def test_search_ragged_groups_match_oracle(sm, oracle, P):
    """325 blocks without importances: a full group of 256 blocks and a ragged one of 69,
    whose last coefficient word (P = 3) is part filled, bit for bit against the oracle."""
    import torch
    M, K = 5, 520
    say("search ragged groups", P, M * K // 8)
    W = _search_case(M, K, f"rag{P}")
    ref = oracle.search_matrix(W, P, -4, None)
    got = sm.search(torch.from_numpy(W).cuda(), P, -4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got["seeds"].cpu().view(torch.int16).numpy().view(np.uint16), ref["seeds"])
    np.testing.assert_array_equal(got["coefs"].cpu().view(torch.int16).numpy().view(np.uint16), ref["coefs"])
    np.testing.assert_array_equal(got["codes"].cpu().numpy(), ref["codes"])
    np.testing.assert_array_equal(got["err"].cpu().numpy().view(np.uint64), ref["err"].view(np.uint64))


@pytest.mark.parametrize("P", [4, 3])
def test_search_recovers_a_seed_coded_matrix(sm, oracle, P):
    """A matrix decoded from random streams is an exact fit: the GPU encoding decodes back
    to it bit for bit (GPU reconstruct) with zero error in every block."""
    import torch
    M, K = 5, 64
    say("search planted matrix", P)
    mat = synth.seed_matrix(synth.config_seed(8), f"pl{P}", M, K, P)
    W = oracle.reconstruct_f32(mat, M, K, P)
    got = sm.search(torch.from_numpy(W).cuda(), P, -4)
    torch.cuda.synchronize()
    assert float(got["err"].abs().max()) == 0.0
    Wg = sm.reconstruct(got, M, K, P)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Wg.cpu().numpy(), W)


# ---------------------------------------------------------------------------------
# Mixed packs: P chosen per expert
# ---------------------------------------------------------------------------------
def _mixed(E, H, I, Ps, tag):
    base = synth.config_seed(10)
    return tuple(synth.seed_matrix_mixed(base, f"{tag}.{n}", *((I, H) if n != "down" else (H, I)), Ps)
                 for n in ("gate", "up", "down"))


def _run_mixed(sm, mats, Ps, ids, w, x, E, H, I):
    import torch
    xt, x32 = bf16_tensor(x)
    mask = sm.p4_mask(Ps, "cuda")
    y = sm.moe_mixed(torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), xt, E, H, I, mask,
                     *[dev(m) for m in mats], Ps=Ps)
    torch.cuda.synchronize()
    return y.cpu().numpy(), x32


@pytest.mark.parametrize("T", [1, 5, 600])
def test_moe_mixed_matches_oracle(sm, oracle, T):
    """P3 and P4 experts in one stack: decode (T = 5), one token (T = 1) and the prefill
    path (T = 600, 150 tokens per expert) against the oracle's mixed layer."""
    E, H, I, k = 8, 256, 128, 2
    Ps = [4, 3, 3, 4, 3, 4, 4, 3]
    say("moe mixed", T)
    mats = _mixed(E, H, I, Ps, "mxg")
    base = synth.config_seed(10)
    ids, w = synth.route_topk(base, f"mxg.r{T}", T, E, k)
    x = synth.normal_f32(base, f"mxg.x{T}", (T, H))
    y, x32 = _run_mixed(sm, mats, Ps, ids, w, x, E, H, I)
    rows = range(T) if T <= 8 else (0, 17, T // 2, T - 1)
    for t in rows:
        ref = oracle.moe_mixed(ids[t:t + 1], w[t:t + 1], x32[t:t + 1], E, H, I, Ps, *mats)
        assert rel_l2(y[t], ref[0]) <= 1e-2, t


def test_moe_mixed_full_size_sampled(sm, oracle):
    E, H, I, k, T = 100, 2048, 1024, 8, 16
    Ps = [4 if v else 3 for v in (synth.uniform_u64(synth.config_seed(10), "mix.P", E) & np.uint64(1))]
    say("moe mixed full size", sum(p == 4 for p in Ps))
    mats = _mixed(E, H, I, Ps, "mxf")
    base = synth.config_seed(10)
    ids, w = synth.route_topk(base, "mxf.r", T, E, k)
    x = synth.normal_f32(base, "mxf.x", (T, H))
    y, x32 = _run_mixed(sm, mats, Ps, ids, w, x, E, H, I)
    for t in (0, 9, 15):
        ref = oracle.moe_mixed(ids[t:t + 1], w[t:t + 1], x32[t:t + 1], E, H, I, Ps, *mats)
        assert rel_l2(y[t], ref[0]) <= 1e-2, t


@pytest.mark.parametrize("P,T", [(4, 16), (3, 16), (3, 1)])
def test_moe_mixed_with_one_p_is_the_uniform_layer(sm, P, T):
    """A mixed pack whose experts all have one P is that P's uniform pack: bit-identical
    outputs from the mixed entry point and the uniform one."""
    E, H, I, k = 100, 2048, 1024, 8
    say("moe mixed all-P vs uniform", P, T)
    gate, up, down, ids, w, x = moe_case(T, E, H, I, P, k, 2, f"mxu{P}")
    y_uni, _ = run_moe(sm, gate, up, down, ids, w, x, E, H, I, P)
    y_mix, _ = _run_mixed(sm, (gate, up, down), [P] * E, ids, w, x, E, H, I)
    assert np.array_equal(y_uni.view(np.uint32), y_mix.view(np.uint32))


def test_moe_mixed_graph_replays_match_eager(sm):
    """The mixed layer with a side stream (its P = 3 launches forked onto the caller's
    second stream and joined back) captured in a HIP graph: every replay, with eager work
    and synchronisations between replays, gives the eager single-stream result bit for
    bit."""
    import torch
    E, H, I, k, T = 100, 2048, 1024, 8, 16
    Ps = [4 if v else 3 for v in (synth.uniform_u64(synth.config_seed(10), "mix.P", E) & np.uint64(1))]
    say("moe mixed graph replay", sum(p == 4 for p in Ps))
    mats = _mixed(E, H, I, Ps, "mxr")
    base = synth.config_seed(10)
    ids, w = synth.route_topk(base, "mxr.r", T, E, k)
    x = synth.normal_f32(base, "mxr.x", (T, H))
    y_ref, _ = _run_mixed(sm, mats, Ps, ids, w, x, E, H, I)
    g, u, d = (dev(m) for m in mats)
    mask = sm.p4_mask(Ps, "cuda")
    ids_t, w_t = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    xt, _ = bf16_tensor(x)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(sm.moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    two = sm.SideStream()
    call = lambda ids_in, y_out: sm.moe_mixed(ids_in, w_t, xt, E, H, I, mask, g, u, d, Ps=Ps,
                                              y=y_out, workspace=ws, side=two)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(ids_t, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    G = torch.cuda.CUDAGraph()
    with torch.cuda.graph(G):
        call(ids_t, y)
    other = torch.from_numpy(np.roll(ids, 1, axis=0)).cuda()
    for rep in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xFF)
        G.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), rep
        call(other, torch.empty_like(y))
        torch.cuda.synchronize()
