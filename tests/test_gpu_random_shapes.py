"""GPU parity over seeded random shapes: products and whole layers at sizes, coefficient
counts, exponent biases and batch sizes drawn from a fixed counter-based stream, each
compared with the oracle.  The hand-picked shapes of the other tests cover the known
boundaries; these cover the combinations between them (ragged rows and K, vector and
per-block stream paths, one-token, decode and prefill kernels, empty experts)."""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

BASE = synth.config_seed(61)


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def rel_l2(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def _dev(mat):
    import torch
    return {
        "seeds": torch.from_numpy(mat["seeds"].view(np.int16).copy()).view(torch.uint16).cuda(),
        "coefs": torch.from_numpy(mat["coefs"].view(np.int16).copy()).view(torch.uint16).cuda(),
        "codes": torch.from_numpy(mat["codes"].copy()).cuda(),
        "exp_bias": torch.from_numpy(mat["exp_bias"].copy()).cuda(),
        "exp_bias_host": mat["exp_bias"].copy(),
    }


def _draw(tag, n, lo, hi):
    return [int(v) for v in synth.uniform_ints(BASE, tag, n, lo, hi)]


N_GEMV, N_MOE = 24, 12
G_M = _draw("g.M", N_GEMV, 1, 300)
# K: a multiple of 64 (vector stream path) for even cases, of 8 (per-block path) for odd
G_K = [64 * a if i % 2 == 0 else 8 * b
       for i, (a, b) in enumerate(zip(_draw("g.K64", N_GEMV, 1, 40), _draw("g.K8", N_GEMV, 1, 300)))]
G_P = _draw("g.P", N_GEMV, 3, 4)
G_N = _draw("g.N", N_GEMV, 1, 80)
G_EB = _draw("g.eb", N_GEMV, -30, 10)
G_BF = _draw("g.bf", N_GEMV, 0, 1)


@pytest.mark.parametrize("i", range(N_GEMV))
def test_random_gemv_matches_oracle(oracle, i):
    import torch
    from pseudo_random_weight_amd import seedmm as sm
    M, K, P, N, eb, bf = G_M[i], G_K[i], G_P[i], G_N[i], G_EB[i], G_BF[i]
    say("random gemv", i, M, K, P, N, eb, "bf16" if bf else "fp32")
    mat = synth.seed_matrix(BASE, f"g{i}", M, K, P, 1, exp_bias=eb)
    x = synth.normal_f32(BASE, f"gx{i}", (N, K))
    if bf:
        bits = synth.bf16_bits(x)
        x = synth.bf16_bits_to_f32(bits)
        xt = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    else:
        xt = torch.from_numpy(x).cuda()
    y = sm.gemv_ex(_dev(mat), xt, M, K, P)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert rel_l2(y, oracle.gemv(mat, x, M, K, P)) <= (1e-2 if bf else 1e-5)
    if bf:
        # bf16 activations: the kernels multiply the bf16 (nearest-even) weights with
        # fp32 sums
        Wb = synth.bf16_bits_to_f32(oracle.reconstruct_bf16(mat, M, K, P)).astype(np.float64)
        assert rel_l2(y, x.astype(np.float64) @ Wb.T) <= 1e-5


# Case i % 4: 0 = one token, H and I multiples of 64 (vector path); 1 and 3 = H and I
# multiples of 8 (per-block path), 2..200 tokens; 2 = H and I multiples of 256 and
# 300..600 tokens, so most such calls have >= 64 tokens per expert (LDS-tile prefill)
L_E = _draw("m.E", N_MOE, 2, 20)
_H64, _H8, _H256 = _draw("m.H64", N_MOE, 1, 8), _draw("m.H8", N_MOE, 2, 48), _draw("m.H256", N_MOE, 1, 2)
_I64, _I8, _I256 = _draw("m.I64", N_MOE, 1, 8), _draw("m.I8", N_MOE, 2, 48), _draw("m.I256", N_MOE, 1, 2)
L_H = [(64 * _H64[i], 8 * _H8[i], 256 * _H256[i], 8 * _H8[i])[i % 4] for i in range(N_MOE)]
L_I = [(64 * _I64[i], 8 * _I8[i], 256 * _I256[i], 8 * _I8[i])[i % 4] for i in range(N_MOE)]
L_K = _draw("m.k", N_MOE, 1, 8)
_T, _TP = _draw("m.T", N_MOE, 2, 200), _draw("m.TP", N_MOE, 300, 600)
L_T = [(1, _T[i], _TP[i], _T[i])[i % 4] for i in range(N_MOE)]
L_P = _draw("m.P", N_MOE, 3, 4)


@pytest.mark.parametrize("i", range(N_MOE))
def test_random_moe_matches_oracle(oracle, i):
    import torch
    from pseudo_random_weight_amd import seedmm as sm
    E, H, I, P, T = L_E[i], L_H[i], L_I[i], L_P[i], L_T[i]
    k = min(L_K[i], E)
    say("random moe", i, E, H, I, P, k, T)
    # per-matrix biases where SiLU bends (gate outputs of order one)
    mats = [synth.seed_matrix(BASE, f"m{i}.{n}", *((I, H) if n != "down" else (H, I)), P, E,
                              exp_bias=synth.uniform_ints(BASE, f"m{i}.{n}.eb", E, lo, lo + 2))
            for n, lo in (("gate", -22), ("up", -21), ("down", -20))]
    ids, w = synth.route_topk(BASE, f"m{i}.r", T, E, k)
    bits = synth.bf16_bits(synth.normal_f32(BASE, f"m{i}.x", (T, H)))
    x32 = synth.bf16_bits_to_f32(bits)
    xt = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    y = sm.moe(torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), xt, E, H, I, P,
               *[_dev(m) for m in mats])
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle.moe(ids, w, x32, E, H, I, P, *mats)
    for t in range(T):
        assert rel_l2(y[t], ref[t]) <= 1e-2, t


N_MIX = 8
X_E = _draw("x.E", N_MIX, 2, 16)
X_H = [8 * v for v in _draw("x.H8", N_MIX, 2, 40)]
X_I = [8 * v for v in _draw("x.I8", N_MIX, 2, 40)]
X_K = _draw("x.k", N_MIX, 1, 8)
_XT, _XTP = _draw("x.T", N_MIX, 2, 100), _draw("x.TP", N_MIX, 300, 500)
X_T = [(1, _XT[i], _XTP[i], _XT[i])[i % 4] for i in range(N_MIX)]   # one token, decode, prefill


@pytest.mark.parametrize("i", range(N_MIX))
def test_random_mixed_pack_matches_oracle(oracle, i):
    """Mixed packs (P drawn per expert), per-expert biases in SiLU's curved range."""
    import torch
    from pseudo_random_weight_amd import seedmm as sm
    E, H, I, T = X_E[i], X_H[i], X_I[i], X_T[i]
    k = min(X_K[i], E)
    Ps = [int(p) for p in synth.uniform_ints(BASE, f"x{i}.P", E, 3, 4)]
    say("random mixed", i, E, H, I, k, T, "".join(map(str, Ps)))
    mats = [synth.seed_matrix_mixed(BASE, f"x{i}.{n}", *((I, H) if n != "down" else (H, I)), Ps,
                                    exp_bias=synth.uniform_ints(BASE, f"x{i}.{n}.eb", E, lo, lo + 2))
            for n, lo in (("gate", -22), ("up", -21), ("down", -20))]
    ids, w = synth.route_topk(BASE, f"x{i}.r", T, E, k)
    bits = synth.bf16_bits(synth.normal_f32(BASE, f"x{i}.x", (T, H)))
    x32 = synth.bf16_bits_to_f32(bits)
    xt = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    y = sm.moe_mixed(torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), xt, E, H, I,
                     sm.p4_mask(Ps, "cuda"), *[_dev(m) for m in mats], Ps=Ps)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle.moe_mixed(ids, w, x32, E, H, I, Ps, *mats)
    for t in range(T):
        assert rel_l2(y[t], ref[t]) <= 1e-2, t
