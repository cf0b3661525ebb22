"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each checks the oracle against a
closed form, an exhaustive invariant, a brute-force re-derivation from a different
formulation (bit streams from the characteristic polynomial), a library routine
(numpy float64 products), or a number the pages print (tests/golden/pages_facts.json).
"""
import json
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def facts():
    with open(GOLDEN) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


# ---------------------------------------------------------------------------
# Bit-stream view of the register, derived from its characteristic polynomial
# x^16 + x^14 + x^13 + x^11 + 1: stream bit x_n = x_{n-16} ^ x_{n-14} ^ x_{n-13} ^ x_{n-11},
# the first 16 bits are the seed (most significant first), and state s_t is the
# 16-bit window x_t .. x_{t+15}.  A formulation independent of the oracle's
# step-the-state code.
# ---------------------------------------------------------------------------
def stream_bits(seeds: np.ndarray, nbits: int) -> np.ndarray:
    seeds = np.asarray(seeds, dtype=np.int64)
    x = np.zeros((seeds.size, nbits), dtype=np.int64)
    for k in range(16):
        x[:, k] = (seeds >> (15 - k)) & 1
    for n in range(16, nbits):
        x[:, n] = x[:, n - 16] ^ x[:, n - 14] ^ x[:, n - 13] ^ x[:, n - 11]
    return x


def windows(bits: np.ndarray, t: int) -> np.ndarray:
    w = np.zeros(bits.shape[0], dtype=np.int64)
    for k in range(16):
        w = (w << 1) | bits[:, t + k]
    return w


ALL_SEEDS = np.arange(65536, dtype=np.int64)


@pytest.fixture(scope="module")
def all_states(oracle):
    """Oracle states s_1..s_32 for every 16-bit seed (65536 x 32)."""
    out = np.zeros((65536, 32), dtype=np.int64)
    for s in range(65536):
        out[s] = oracle.states(s, 32)
    return out


def test_period_is_65535_and_visits_every_nonzero_state(oracle):
    # "all 65,535 seeds" (model card P4, 'How it works'): a maximal-length register
    orbit = oracle.states(1, 65535).astype(np.int64)
    assert orbit[-1] == 1                      # back at the seed after 65,535 steps
    assert len(np.unique(orbit)) == 65535       # every nonzero state exactly once
    assert 0 not in set(orbit.tolist())
    assert facts()["nonzero_seeds"] == 65535


def test_seed_zero_is_a_fixed_point(oracle):
    assert np.all(oracle.states(0, 32) == 0)


def test_states_are_windows_of_one_stream(all_states):
    # model/blog 'LFSR is free': states become shifts of one 64-bit word
    bits = stream_bits(ALL_SEEDS, 48)
    for t in range(1, 33):
        np.testing.assert_array_equal(all_states[:, t - 1], windows(bits, t))
    # and the 48-bit word seed<<32 | next32 holds every s_t at bit offset 32 - t
    word = (ALL_SEEDS << 32) | (all_states[:, 15] << 16) | all_states[:, 31]
    for t in range(0, 33):
        np.testing.assert_array_equal((word >> (32 - t)) & 0xFFFF,
                                      ALL_SEEDS if t == 0 else all_states[:, t - 1])


def test_following_bits_are_gf2_linear_in_the_seed(all_states):
    # 'LFSR is free': the 24 or 32 bits that follow any seed are a linear function of it
    next32 = (all_states[:, 15] << 16) | all_states[:, 31]
    basis = next32[1 << np.arange(16)]
    pred = np.zeros(65536, dtype=np.int64)
    for i in range(16):
        pred ^= np.where((ALL_SEEDS >> i) & 1, basis[i], 0)
    np.testing.assert_array_equal(next32, pred)
    next24 = (all_states[:, 15] << 8) | (all_states[:, 23] & 0xFF)
    np.testing.assert_array_equal(next24, pred >> 8)


def test_basis_value_matches_the_mantissa_bit_insert(oracle):
    # 'LFSR is free', two-operation states: 16 state bits inserted in the mantissa of 1.0
    # give 1 + state/65536; the basis value is the affine map 2*(1 + s/65536) - 3 =
    # (s - 32768)/32768 of it (offset 32768, the 2^16 folded into the exponent).
    s = np.arange(65536, dtype=np.uint32)
    f = (np.uint32(0x3F800000) | (s << np.uint32(7))).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(f, 1.0 + s / 65536.0)
    # weight 0 of a block with c = (1, 0, 0, 0), code 0, exp_bias 0 is the basis value of
    # s_1 = step(seed); as the seed runs over all nonzero states so does s_1
    bits = stream_bits(ALL_SEEDS[1:], 17)
    s1 = windows(bits, 1)
    f1 = (np.uint32(0x3F800000) | (s1.astype(np.uint32) << np.uint32(7))).view(np.float32)
    expect = 2.0 * f1.astype(np.float64) - 3.0
    got = np.array([oracle.block(int(sd), [1, 0, 0, 0], 4, 0, 0)[0] for sd in ALL_SEEDS[1:]])
    np.testing.assert_array_equal(got.astype(np.float64), expect)


def test_nibble_sign_extension_table(oracle):
    # 'LFSR is free', convert-free coefficients: (q ^ 8) - 8 sign-extends a nibble
    table = [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]
    for q in range(16):
        for P in (3, 4):
            for j in range(P):
                words = np.zeros(4, dtype=np.uint16)
                n = 1 * P + j                          # block 1, coefficient j
                words[n >> 2] = q << (4 * (n & 3))
                assert oracle.coef(words, 1, P, j) == table[q] == (q ^ 8) - 8


def test_nibble_stream_and_code_packing(oracle):
    rng = np.random.default_rng(7)
    for P in (3, 4):
        nib = rng.integers(0, 16, size=64 * P)
        words = np.zeros((nib.size + 3) // 4, dtype=np.uint16)
        for n, q in enumerate(nib):
            words[n // 4] |= np.uint16(int(q) << (4 * (n % 4)))
        for b in range(64):
            for j in range(P):
                q = int(nib[b * P + j])
                assert oracle.coef(words, b, P, j) == (q - 16 if q >= 8 else q)
    codes_nib = rng.integers(0, 16, size=64)
    cb = np.array([codes_nib[2 * i] | (codes_nib[2 * i + 1] << 4) for i in range(32)], dtype=np.uint8)
    for b in range(64):
        assert oracle.code(cb, b) == codes_nib[b]


def test_size_identities_from_the_pages(oracle):
    F = facts()
    for (M, K) in [(256, 512), (768, 2048), (2048, 768), (1024, 2048), (2048, 1024)]:
        for P, bpw in [(4, F["bits_per_weight_P4"]), (3, F["bits_per_weight_P3"])]:
            a, b, c = oracle.stream_bytes(M, K, P)
            assert (a + b + c) * 8 == bpw * M * K
    # 4 int4 coefs + 16-bit seed + 4-bit code per 8 weights = 4.5 bpw, the same bits as
    # affine Q4 group 64 -- the reason p4mx and the Q4 pack are both 26.53 GB
    assert (16 + 4 * 4 + 4) / 8 == F["bits_per_weight_P4"] == F["affine_q4_g64_bits"]
    assert (16 + 3 * 5 + 4) / 8 == F["bits_per_weight_P3_5bit_coefs"]
    # 120.8 B expert weights -> 68.0 GB (P4) and 60.4 GB (P3); one code byte per block
    # instead of a nibble would give 5.0 bits and 75.5 GB instead
    gb4 = F["qwen_expert_weights"] * F["bits_per_weight_P4"] / 8 / 1e9
    gb3 = F["qwen_expert_weights"] * F["bits_per_weight_P3"] / 8 / 1e9
    assert round(gb4, 1) == F["qwen_P4_expert_GB"]
    assert round(gb3, 1) == F["qwen_P3_expert_GB"]
    assert round(F["qwen_expert_weights"] * 5.0 / 8 / 1e9, 1) != F["qwen_P4_expert_GB"]


def test_exponent_multiplies(oracle):
    # blog 'Attempt one': the dequantization must multiply by 2^e, not divide
    rng = np.random.default_rng(3)
    for _ in range(50):
        seed = int(rng.integers(1, 65536))
        c = [int(v) for v in rng.integers(-8, 8, size=4)]
        code_ = int(rng.integers(0, 15))
        w0 = oracle.block(seed, c, 4, code_, -4)
        w1 = oracle.block(seed, c, 4, code_ + 1, -4)
        np.testing.assert_array_equal(w1, 2.0 * w0)
        wb = oracle.block(seed, c, 4, code_, -3)
        np.testing.assert_array_equal(wb, w1)


def _brute_force_matrix(mat, M, K, P):
    """W from the bit-stream formulation with Python integers (no oracle code)."""
    nblk = M * K // 8
    seeds = mat["seeds"].astype(np.int64)
    bits = stream_bits(seeds[:nblk], 16 + 8 * P + 16)
    nibbles = []
    for wd in mat["coefs"].astype(np.int64):
        nibbles += [(wd >> (4 * r)) & 15 for r in range(4)]
    codes = []
    for byte in mat["codes"].astype(np.int64):
        codes += [byte & 15, byte >> 4]
    eb = int(mat["exp_bias"][0])
    W = np.zeros((M, K), dtype=np.float64)
    for b in range(nblk):
        m, kb = divmod(b, K // 8)
        c = [nibbles[b * P + j] - 16 * (nibbles[b * P + j] >= 8) for j in range(P)]
        states = [int(windows(bits[b:b + 1], t)[0]) for t in range(1, 8 * P + 1)]
        for i in range(8):
            acc = sum(c[j] * (states[i * P + j] - 32768) for j in range(P))
            W[m, 8 * kb + i] = acc * 2.0 ** (codes[b] + eb - 15)
    return W


@pytest.mark.parametrize("P", [3, 4])
@pytest.mark.parametrize("M,K", [(3, 24), (2, 64), (5, 8)])
def test_reconstruct_brute_force_tiny(oracle, P, M, K):
    mat = synth.seed_matrix(synth.config_seed(90 + P), f"tiny{M}x{K}", M, K, P)
    mat["exp_bias"][:] = -2
    Wb = _brute_force_matrix(mat, M, K, P)
    Wo = oracle.reconstruct_f32(mat, M, K, P)
    np.testing.assert_array_equal(Wo.astype(np.float64), Wb)


def test_reconstructed_weights_are_exact_and_bounded(oracle):
    mat = synth.seed_matrix(synth.config_seed(0), "W", 64, 512, 4)
    W = oracle.reconstruct_f32(mat, 64, 512, 4).astype(np.float64)
    codes = np.repeat(np.stack([mat["codes"] & 15, mat["codes"] >> 4], 1).reshape(-1), 8)
    ints = W.reshape(-1) * 2.0 ** (15 - (codes.astype(np.int64) - 4))
    assert np.all(ints == np.round(ints))
    assert np.max(np.abs(ints)) <= 2 ** 20


def test_bf16_rounding_is_nearest_even(oracle):
    cases = {1.0: 0x3F80, 1.0 + 2 ** -8: 0x3F80, 1.0 + 3 * 2 ** -8: 0x3F82,
             1.0 + 2 ** -8 + 2 ** -20: 0x3F81, -2.5: 0xC020, 65535.0: 0x4780, 3.0: 0x4040}
    for f, bits in cases.items():
        assert oracle.f32_to_bf16(f) == bits, f
    mat = synth.seed_matrix(synth.config_seed(0), "W", 32, 256, 4)
    Wf = oracle.reconstruct_f32(mat, 32, 256, 4)
    Wb = oracle.reconstruct_bf16(mat, 32, 256, 4)
    # nearest: |bf16 - w| <= half an ulp of bf16 at w; and equal to numpy's RNE
    back = synth.bf16_bits_to_f32(Wb).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(Wf.astype(np.float64)), 1e-30))) - 7)
    assert np.all(np.abs(back - Wf) <= ulp / 2 + 0.0)
    np.testing.assert_array_equal(Wb, synth.bf16_bits(Wf))


@pytest.mark.parametrize("P", [3, 4])
def test_gemv_equals_float64_matmul(oracle, P):
    M, K, N = 64, 512, 3
    mat = synth.seed_matrix(synth.config_seed(0), f"g{P}", M, K, P)
    x = synth.normal_f32(synth.config_seed(0), "x", (N, K))
    W = oracle.reconstruct_f32(mat, M, K, P).astype(np.float64)
    ref = (x.astype(np.float64) @ W.T)
    y = oracle.gemv(mat, x, M, K, P)
    np.testing.assert_allclose(y, ref.astype(np.float32), rtol=1e-6, atol=0)


def test_gemv_one_hot_returns_a_column(oracle):
    M, K = 48, 256
    mat = synth.seed_matrix(synth.config_seed(0), "oh", M, K, 4)
    W = oracle.reconstruct_f32(mat, M, K, 4)
    for k in [0, 7, 8, 131, 255]:
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        np.testing.assert_array_equal(oracle.gemv(mat, x, M, K, 4)[0], W[:, k])


def _np_expert(Wg, Wu, Wd, x):
    g = x @ Wg.T
    u = x @ Wu.T
    h = g / (1.0 + np.exp(-g)) * u
    return h @ Wd.T


@pytest.mark.parametrize("P", [3, 4])
def test_expert_equals_float64_composition(oracle, P):
    H, I, T = 128, 64, 3
    base = synth.config_seed(1)
    gate = synth.seed_matrix(base, "gate", I, H, P)
    up = synth.seed_matrix(base, "up", I, H, P)
    down = synth.seed_matrix(base, "down", H, I, P)
    x = synth.bf16_bits_to_f32(synth.bf16_bits(synth.normal_f32(base, "x", (T, H))))
    Wg = oracle.reconstruct_f32(gate, I, H, P).astype(np.float64)
    Wu = oracle.reconstruct_f32(up, I, H, P).astype(np.float64)
    Wd = oracle.reconstruct_f32(down, H, I, P).astype(np.float64)
    ref = _np_expert(Wg, Wu, Wd, x.astype(np.float64))
    got = oracle.expert(gate, up, down, x, H, I, P)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-9 * np.abs(ref).max())


def _small_moe(P, E=5, H=64, I=32, T=6, k=2, cfg=2):
    base = synth.config_seed(cfg)
    gate = synth.seed_matrix(base, "gate", I, H, P, E)
    up = synth.seed_matrix(base, "up", I, H, P, E)
    down = synth.seed_matrix(base, "down", H, I, P, E)
    x = synth.bf16_bits_to_f32(synth.bf16_bits(synth.normal_f32(base, "x", (T, H))))
    ids, w = synth.route_topk(base, "router", T, E, k)
    return gate, up, down, x, ids, w


@pytest.mark.parametrize("P", [3, 4])
def test_moe_equals_weighted_sum_of_experts(oracle, P):
    E, H, I, T, k = 5, 64, 32, 6, 2
    gate, up, down, x, ids, w = _small_moe(P, E, H, I, T, k)
    y = oracle.moe(ids, w, x, E, H, I, P, gate, up, down)
    ref = np.zeros((T, H))
    for e in range(E):
        Wg = oracle.reconstruct_f32({kk: v for kk, v in _slice(gate, I, H, P, e).items()}, I, H, P)
        Wu = oracle.reconstruct_f32(_slice(up, I, H, P, e), I, H, P)
        Wd = oracle.reconstruct_f32(_slice(down, H, I, P, e), H, I, P)
        out = _np_expert(Wg.astype(np.float64), Wu.astype(np.float64), Wd.astype(np.float64),
                         x.astype(np.float64))
        for t in range(T):
            for s in range(k):
                if ids[t, s] == e:
                    ref[t] += float(w[t, s]) * out[t]
    np.testing.assert_allclose(y, ref.astype(np.float32), rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def _slice(mat, M, K, P, e):
    nblk = M * K // 8
    cw, cb = nblk * P // 4, nblk // 2
    return {"seeds": mat["seeds"][e * nblk:(e + 1) * nblk],
            "coefs": mat["coefs"][e * cw:(e + 1) * cw],
            "codes": mat["codes"][e * cb:(e + 1) * cb],
            "exp_bias": mat["exp_bias"][e:e + 1]}


def test_moe_top1_weight1_is_the_expert(oracle):
    E, H, I, T = 4, 64, 32, 5
    gate, up, down, x, _, _ = _small_moe(4, E, H, I, T, 1)
    ids = np.full((T, 1), 2, dtype=np.int32)
    w = np.ones((T, 1), dtype=np.float32)
    y = oracle.moe(ids, w, x, E, H, I, 4, gate, up, down)
    ref = oracle.expert(gate, up, down, x, H, I, 4, e=2)
    np.testing.assert_array_equal(y, ref.astype(np.float32))


def test_moe_token_permutation_equivariance(oracle):
    E, H, I, T, k = 5, 64, 32, 6, 2
    gate, up, down, x, ids, w = _small_moe(4, E, H, I, T, k)
    y = oracle.moe(ids, w, x, E, H, I, 4, gate, up, down)
    perm = np.array([3, 0, 5, 1, 4, 2])
    yp = oracle.moe(ids[perm], w[perm], x[perm], E, H, I, 4, gate, up, down)
    np.testing.assert_array_equal(yp, y[perm])


def test_moe_does_not_depend_on_the_thread_count(oracle):
    """Every row is summed in a fixed order, so the oracle's result is the same on one
    thread as on many (the benchmark times it both ways)."""
    E, H, I, T, k = 6, 128, 64, 9, 3
    gate, up, down, x, ids, w = _small_moe(4, E, H, I, T, k)
    n = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        y1 = oracle.moe(ids, w, x, E, H, I, 4, gate, up, down)
    finally:
        oracle.set_num_threads(n)
    yn = oracle.moe(ids, w, x, E, H, I, 4, gate, up, down)
    np.testing.assert_array_equal(y1, yn)


def test_moe_rejects_out_of_range_ids(oracle):
    E, H, I, T, k = 3, 64, 32, 2, 1
    gate, up, down, x, _, _ = _small_moe(4, E, H, I, T, k)
    with pytest.raises(ValueError):
        oracle.moe(np.array([[0], [3]], dtype=np.int32), np.ones((2, 1), np.float32), x,
                   E, H, I, 4, gate, up, down)


@pytest.mark.parametrize("P", [4, 3])
def test_planted_seed_is_recovered_by_exhaustive_search(oracle, P):
    # model card P4 'How it works': the search tries all 65,535 seeds per block.  A block
    # synthesised from (seed*, c*, code*) is an exact fit, so the search must return a
    # block bit-identical to it, with seed*.  c* has an odd entry (no halving to code*+1)
    # and an entry outside [-4, 3] (no doubling to code*-1), so (c*, code*) is the only
    # exact encoding with seed*.
    rng = np.random.default_rng(11 + P)
    for trial in range(2):
        while True:
            c = [int(v) for v in rng.integers(-8, 8, size=P)]
            if any(v % 2 for v in c) and any(v >= 4 or v <= -5 for v in c) and \
                    sum(v != 0 for v in c) >= 2:
                break
        seed = int(rng.integers(1, 65536))
        code_ = int(rng.integers(0, 16))
        w = oracle.block(seed, c, P, code_, -4).astype(np.float64)
        s2, c2, code2, err = oracle.search_block(w, -4, P)
        assert err == 0.0
        assert (s2, c2, code2) == (seed, c, code_)
        np.testing.assert_array_equal(oracle.block(s2, c2, P, code2, -4), w.astype(np.float32))


def test_search_finds_nearest_for_a_perturbed_block(oracle):
    # a block off by a tiny amount still comes back to its planted seed (nearest fit)
    seed, c, code_ = 4242, [5, -3, 0, 7], 9
    w = oracle.block(seed, c, 4, code_, -4).astype(np.float64)
    w = w + 1e-3 * np.abs(w).max() * np.sin(np.arange(8))
    s2, c2, code2, err = oracle.search_block(w, -4, 4)
    assert (s2, c2, code2) == (seed, c, code_)
    assert err > 0


def _all_states(P):
    """States s_1..s_8P of every seed 1..65535, by a vectorised register written here
    from the polynomial x^16 + x^14 + x^13 + x^11 + 1 (shift left, feedback into bit 0)."""
    s = np.arange(1, 65536, dtype=np.uint32)
    out = np.empty((65535, 8 * P), dtype=np.int64)
    for t in range(8 * P):
        fb = ((s >> 15) ^ (s >> 13) ^ (s >> 12) ^ (s >> 10)) & 1
        s = ((s << 1) | fb) & 0xFFFF
        out[:, t] = s
    return out


def _brute_force_search(w8, P, exp_bias, d8):
    """Every seed's least-squares coefficients (numpy solve), every code's rounded and
    clamped coefficients, and the weighted squared error of each candidate."""
    U = (_all_states(P) - 32768).astype(np.float64).reshape(65535, 8, P)
    d = np.ones(8) if d8 is None else np.asarray(d8, dtype=np.float64)
    A = np.einsum("sij,i,sik->sjk", U, d, U)
    r = np.einsum("sij,i,i->sj", U, d, w8)
    full = np.linalg.matrix_rank(A) == P       # singular systems have no LS solution
    alpha = np.zeros((65535, P))
    alpha[full] = np.linalg.solve(A[full], r[full][..., None])[..., 0]
    best = (np.inf, None, None)
    for code in range(16):
        sc = 2.0 ** (code + exp_bias - 15)
        c = np.clip(np.rint(alpha / sc), -8, 7)
        v = np.einsum("sij,sj->si", U, c)
        err = ((w8[None, :] - sc * v) ** 2 * d[None, :]).sum(axis=1)
        err[~full] = np.inf
        i = int(np.argmin(err))
        if err[i] < best[0]:
            best = (float(err[i]), i + 1, code)
    return best


@pytest.mark.parametrize("weighted", [False, True])
def test_search_picks_the_brute_force_minimum(oracle, weighted):
    # an independent re-derivation of the search (numpy LFSR, batched solve): the oracle's
    # choice reaches the smallest squared error over all 65,535 x 16 candidates
    rng = np.random.default_rng(77 + weighted)
    for P in (4, 3):
        w8 = rng.standard_normal(8) * 0.05
        d8 = rng.uniform(0.1, 3.0, 8) if weighted else None
        s2, c2, code2, err = oracle.search_block(w8, -4, P, d8)
        ref_err, ref_seed, ref_code = _brute_force_search(w8, P, -4, d8)
        assert err == pytest.approx(ref_err, rel=1e-9, abs=1e-300)
        assert (s2, code2) == (ref_seed, ref_code)
        # the reported error is the error of the returned encoding
        blk = oracle.block(s2, c2, P, code2, -4).astype(np.float64)
        d = np.ones(8) if d8 is None else d8
        assert err == pytest.approx(float((d * (w8 - blk) ** 2).sum()), rel=1e-12)


def test_weighted_search_with_unit_weights_is_the_unweighted_search(oracle):
    rng = np.random.default_rng(5)
    for P in (4, 3):
        w8 = rng.standard_normal(8) * 0.02
        assert oracle.search_block(w8, -4, P, np.ones(8)) == oracle.search_block(w8, -4, P)


@pytest.mark.parametrize("P", [4, 3])
def test_weighted_search_recovers_a_planted_block(oracle, P):
    # an exact encoding has zero error under any positive weighting
    rng = np.random.default_rng(300 + P)
    c = [7, -8, 3, -5][:P]
    seed, code_ = int(rng.integers(1, 65536)), 6
    w = oracle.block(seed, c, P, code_, -4).astype(np.float64)
    s2, c2, code2, err = oracle.search_block(w, -4, P, rng.uniform(0.2, 5.0, 8))
    assert err == 0.0 and (s2, c2, code2) == (seed, c, code_)


@pytest.mark.parametrize("P", [4, 3])
def test_search_matrix_round_trips_a_seed_coded_matrix(oracle, P):
    # W decoded from random streams is an exact fit block by block: encoding it again
    # gives streams that decode to W bit for bit, with zero error everywhere; the P = 3
    # nibble stream (4 blocks per 3 words) and the 2-codes-per-byte stream are packed
    # across block boundaries here
    M, K = 3, 24
    mat = synth.seed_matrix(synth.config_seed(9), f"rt{P}", M, K, P)
    W = oracle.reconstruct_f32(mat, M, K, P)
    enc = oracle.search_matrix(W, P, -4)
    np.testing.assert_array_equal(enc["err"], 0.0)
    np.testing.assert_array_equal(oracle.reconstruct_f32(enc, M, K, P), W)


def _mixed_layer(E, H, I, Ps, tag):
    base = synth.config_seed(10)
    return tuple(synth.seed_matrix_mixed(base, f"{tag}.{n}", *((I, H) if n != "down" else (H, I)), Ps)
                 for n in ("gate", "up", "down"))


def test_moe_mixed_with_one_p_is_the_uniform_layer(oracle):
    E, H, I, T, k = 4, 64, 32, 3, 2
    for P in (4, 3):
        base = synth.config_seed(10)
        mats = [synth.seed_matrix(base, f"u{P}.{n}", *((I, H) if n != "down" else (H, I)), P, E)
                for n in ("gate", "up", "down")]
        ids, w = synth.route_topk(base, f"u{P}.r", T, E, k)
        x = synth.normal_f32(base, f"u{P}.x", (T, H))
        np.testing.assert_array_equal(oracle.moe_mixed(ids, w, x, E, H, I, [P] * E, *mats),
                                      oracle.moe(ids, w, x, E, H, I, P, *mats))


def test_moe_mixed_is_the_slot_sum_of_each_experts_own_ffn(oracle):
    # a stack of P3 and P4 experts: every token's output is the weighted slot sum of the
    # single-expert FFNs, each expert read from its own (un-stacked) streams with its own P
    E, H, I, T, k = 5, 64, 32, 4, 3
    Ps = [4, 3, 3, 4, 3]
    base = synth.config_seed(10)
    parts = {n: [synth.seed_matrix(base, f"mx.{n}.m{e}", *((I, H) if n != "down" else (H, I)), Ps[e])
                 for e in range(E)] for n in ("gate", "up", "down")}
    stacked = [synth.seed_matrix_mixed(base, f"mx.{n}", *((I, H) if n != "down" else (H, I)), Ps)
               for n in ("gate", "up", "down")]
    ids, w = synth.route_topk(base, "mx.r", T, E, k)
    x = synth.normal_f32(base, "mx.x", (T, H))
    y = oracle.moe_mixed(ids, w, x, E, H, I, Ps, *stacked)
    for t in range(T):
        ref = np.zeros(H)
        for s in range(k):
            e = int(ids[t, s])
            ref += float(w[t, s]) * oracle.expert(parts["gate"][e], parts["up"][e], parts["down"][e],
                                                  x[t:t + 1], H, I, Ps[e])[0].astype(np.float64)
        np.testing.assert_allclose(y[t], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_seed_zero_block_is_constant(oracle):
    # every state of seed 0 is 0, so every basis value is -32768 and the 8 weights of the
    # block are 2^(code + exp_bias - 15) * (-32768) * sum_j c_j
    for P, c, code, eb in ((4, [3, -8, 7, 1], 9, -4), (3, [-5, 2, 6, 0], 15, -20), (4, [0, 0, 0, 0], 4, 0)):
        w = oracle.block(0, c, P, code, eb)
        expect = -32768.0 * sum(c[:P]) * 2.0 ** (code + eb - 15)
        assert np.all(w.astype(np.float64) == expect), (w, expect)


def test_silu_in_its_curved_range(oracle):
    # a gate at exp_bias -21 gives gate outputs of order 1: the expert equals the float64
    # composition with silu(z) = z / (1 + e^-z) evaluated where it is far from relu
    H, I, T, P = 256, 64, 4, 4
    base = synth.config_seed(24)
    gate = synth.seed_matrix(base, "cg", I, H, P, exp_bias=-21)
    up = synth.seed_matrix(base, "cu", I, H, P, exp_bias=-19)
    down = synth.seed_matrix(base, "cd", H, I, P, exp_bias=-18)
    x = synth.bf16_bits_to_f32(synth.bf16_bits(synth.normal_f32(base, "cx", (T, H))))
    Wg = oracle.reconstruct_f32(gate, I, H, P).astype(np.float64)
    g = x.astype(np.float64) @ Wg.T
    assert np.mean(np.abs(g) < 4.0) > 0.5 and np.mean(np.abs(g) < 0.5) > 0.05
    # closed-form values of silu at 0, +-1 and +-2
    for z, s in ((0.0, 0.0), (1.0, 0.7310585786300049), (-1.0, -0.2689414213699951),
                 (2.0, 1.7615941559557649), (-2.0, -0.2384058440442351)):
        assert abs(z / (1.0 + np.exp(-z)) - s) < 1e-15
    Wu = oracle.reconstruct_f32(up, I, H, P).astype(np.float64)
    Wd = oracle.reconstruct_f32(down, H, I, P).astype(np.float64)
    ref = _np_expert(Wg, Wu, Wd, x.astype(np.float64))
    got = oracle.expert(gate, up, down, x, H, I, P)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-9 * np.abs(ref).max())
    # relu in place of silu would be far off here (a dropped exponential is caught)
    relu = (np.maximum(g, 0.0) * (x.astype(np.float64) @ Wu.T)) @ Wd.T
    assert np.linalg.norm(relu - ref) > 0.05 * np.linalg.norm(ref)


def test_moe_reads_each_matrix_own_exp_bias(oracle):
    # per-expert biases that differ between gate, up and down: the layer equals the
    # weighted sum of each expert computed from its own three single matrices
    E, H, I, T, k, P = 4, 64, 32, 5, 2, 4
    base = synth.config_seed(25)
    ebs = {"g": [-21, -20, -22, -19], "u": [-18, -22, -20, -21], "d": [-17, -19, -21, -20]}
    gate = synth.seed_matrix(base, "bg", I, H, P, E, exp_bias=ebs["g"])
    up = synth.seed_matrix(base, "bu", I, H, P, E, exp_bias=ebs["u"])
    down = synth.seed_matrix(base, "bd", H, I, P, E, exp_bias=ebs["d"])
    x = synth.bf16_bits_to_f32(synth.bf16_bits(synth.normal_f32(base, "bx", (T, H))))
    ids, w = synth.route_topk(base, "br", T, E, k)
    got = oracle.moe(ids, w, x, E, H, I, P, gate, up, down)
    ref = np.zeros((T, H))
    for t in range(T):
        for s in range(k):
            e = int(ids[t, s])
            mats = []
            for m, (M, K) in ((gate, (I, H)), (up, (I, H)), (down, (H, I))):
                n = M * K // 8
                mats.append(oracle.reconstruct_f32(
                    {"seeds": m["seeds"][e * n:(e + 1) * n].copy(),
                     "coefs": m["coefs"][e * n * P // 4:(e + 1) * n * P // 4].copy(),
                     "codes": m["codes"][e * n // 2:(e + 1) * n // 2].copy(),
                     "exp_bias": m["exp_bias"][e:e + 1].copy()}, M, K, P).astype(np.float64))
            ref[t] += w[t, s] * _np_expert(*mats, x[t:t + 1].astype(np.float64))[0]
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())
