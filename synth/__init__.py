"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module holds no part of the seed-decoding arithmetic: it only draws random
bits and numbers (a counter-based splitmix64 generator, Box-Muller normals, bf16
rounding of the drawn activations) and lays them out in the stream sizes of the
tensor encoding (NAME.seeds U16, NAME.coefs U16, NAME.codes U8, NAME.exp_bias I32,
model card "K2-Horizon-MoVA-36B-A4B - NanoSeedLM p4mx-q4v", section "This upload").

Recipe:
  * seeds uniform in [1, 65535];
  * coefficient nibbles uniform in [-8, 7] and exponent codes uniform in [0, 15];
    both are uniform 4-bit fields, so their packed streams are uniform random words
    and bytes of the stream lengths below;
  * exp_bias = -4 for every matrix, or per matrix values chosen by a test (a stacked
    tensor holds one exp_bias per matrix);
  * activations x ~ N(0, 1) (Box-Muller in float64, then fp32, then bf16 by
    round-to-nearest-even where the workload uses bf16);
  * router logits ~ N(0, 1) fp32 [T][E]; top-k by logit (ties to the lower expert id),
    softmax over the k selected logits; for skewed routing, +1.3 on the logits of a
    seeded random third of the experts (that third then takes about 85% of the choices).
Every tensor draws from its own sub-stream of splitmix64 keyed by (base seed, tag).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "splitmix64", "uniform_u64", "stream_lengths", "seed_matrix", "normal_f32",
    "bf16_bits", "bf16_bits_to_f32", "route_topk", "hot_bias", "config_seed",
    "seed_matrix_mixed", "plant_degenerate", "uniform_ints",
]

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def config_seed(config_id: int) -> int:
    """Base seed of a workload: 0x5EED0000 + config id."""
    return 0x5EED0000 + int(config_id)


def splitmix64(key: int, n: int, start: int = 0) -> np.ndarray:
    """n outputs of splitmix64 with state key, counters start+1 .. start+n (uint64)."""
    with np.errstate(over="ignore"):
        ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(key & 0xFFFFFFFFFFFFFFFF) + ctr * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def _subkey(base: int, tag: str) -> int:
    """Key of the sub-stream for one tensor: splitmix64 of base mixed with the tag."""
    h = 0
    for ch in tag.encode():
        h = (h * 131 + ch) & 0xFFFFFFFFFFFFFFFF
    return int(splitmix64((base * 0x100000001B3) ^ h, 1)[0])


def uniform_u64(base: int, tag: str, n: int) -> np.ndarray:
    return splitmix64(_subkey(base, tag), n)


def stream_lengths(nblk: int, P: int):
    """(seed words, coef words, code bytes) holding nblk blocks of P nibbles each."""
    return nblk, (nblk * P + 3) // 4, (nblk + 1) // 2


def seed_matrix(base: int, tag: str, M: int, K: int, P: int, E: int = 1, exp_bias=-4):
    """Random seed-coded streams for E stacked [M][K] matrices.

    Returns dict(seeds u16, coefs u16, codes u8, exp_bias i32[E]).  exp_bias is one
    value for every matrix or a sequence of E values.  Each expert's streams are whole
    words/bytes (requires (M*K/8)*P % 4 == 0 and (M*K/8) % 2 == 0 when E > 1)."""
    assert K % 8 == 0
    nblk1 = M * (K // 8)
    if E > 1:
        assert (nblk1 * P) % 4 == 0 and nblk1 % 2 == 0
    nblk = nblk1 * E
    ns, nc, nd = stream_lengths(nblk, P)
    r = uniform_u64(base, tag + ".seeds", ns)
    seeds = (r % np.uint64(65535) + np.uint64(1)).astype(np.uint16)
    coefs = (uniform_u64(base, tag + ".coefs", nc) >> np.uint64(48)).astype(np.uint16)
    codes = (uniform_u64(base, tag + ".codes", nd) >> np.uint64(56)).astype(np.uint8)
    eb = np.asarray(exp_bias, dtype=np.int64)
    eb = np.full(E, int(eb), dtype=np.int32) if eb.ndim == 0 else eb.astype(np.int32).reshape(E)
    return {"seeds": seeds, "coefs": coefs, "codes": codes, "exp_bias": eb}


def uniform_ints(base: int, tag: str, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi] (int64)."""
    r = uniform_u64(base, tag, n)
    return (r % np.uint64(hi - lo + 1)).astype(np.int64) + lo


def plant_degenerate(mat: dict, P: int, base: int, tag: str, frac: float = 0.02) -> dict:
    """A copy of `mat` with degenerate blocks planted at seeded random places: seed 0 in
    about `frac` of the blocks, and all-zero coefficient words for about `frac` of the
    aligned groups of 4 blocks (a group's P*4 nibbles fill P whole words).  Returns the
    copy; its 'seed0' and 'zero_groups' entries list the planted block and group indices."""
    out = {k: np.array(v, copy=True) for k, v in mat.items()}
    nblk = out["seeds"].size
    n0 = max(1, int(nblk * frac))
    b0 = np.unique((uniform_u64(base, tag + ".seed0", n0) % np.uint64(nblk)).astype(np.int64))
    out["seeds"][b0] = 0
    ngroups = nblk // 4
    groups = np.zeros(0, dtype=np.int64)
    if ngroups:
        ng = max(1, int(ngroups * frac))
        groups = np.unique((uniform_u64(base, tag + ".zero", ng) % np.uint64(ngroups)).astype(np.int64))
        for g in groups:
            out["coefs"][g * P:(g + 1) * P] = 0
    out["seed0"] = b0
    out["zero_groups"] = groups
    return out


def seed_matrix_mixed(base: int, tag: str, M: int, K: int, Ps, exp_bias=-4):
    """Random streams for len(Ps) stacked [M][K] matrices, matrix e with Ps[e] coefficients
    per block: each matrix generated on its own sub-stream, the streams concatenated in
    matrix order (requires (M*K/8) % 4 == 0).  exp_bias: one value for every matrix or a
    sequence of len(Ps).  Also returns 'P' (int32[E])."""
    assert (M * (K // 8)) % 4 == 0
    eb = np.asarray(exp_bias, dtype=np.int64)
    ebs = [int(eb)] * len(Ps) if eb.ndim == 0 else [int(v) for v in eb.reshape(len(Ps))]
    parts = [seed_matrix(base, f"{tag}.m{e}", M, K, int(P), 1, ebs[e]) for e, P in enumerate(Ps)]
    out = {k: np.concatenate([p_[k] for p_ in parts]) for k in ("seeds", "coefs", "codes", "exp_bias")}
    out["P"] = np.asarray(Ps, dtype=np.int32)
    return out


def normal_f32(base: int, tag: str, shape) -> np.ndarray:
    """N(0,1) samples by Box-Muller in float64, rounded to fp32."""
    n = int(np.prod(shape))
    m = (n + 1) // 2
    r = uniform_u64(base, tag, 2 * m)
    u1 = ((r[:m] >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)
    u2 = (r[m:] >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    rad = np.sqrt(-2.0 * np.log(u1))
    z = np.concatenate([rad * np.cos(2 * np.pi * u2), rad * np.sin(2 * np.pi * u2)])[:n]
    return z.astype(np.float32).reshape(shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, as uint16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def route_topk(base: int, tag: str, T: int, E: int, top_k: int, bias=None):
    """Router logits ~N(0,1) [T][E] (plus bias[E] if given); top-k ids (ties -> lower id)
    and softmax weights."""
    logits = normal_f32(base, tag, (T, E)).astype(np.float64)
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    # stable argsort of -logits keeps the lower id first among equal logits
    order = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    sel = np.take_along_axis(logits, order, axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    w = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def hot_bias(base: int, E: int, hot_frac: float = 1.0 / 3.0, bias: float = 1.3):
    """Router logit offsets that make a seeded random hot set of round(E * hot_frac)
    experts take most router choices: +bias on the hot experts, 0 elsewhere.  With E = 100,
    top-8 and bias 1.3, the hot third takes about 85% of the choices (the documentation
    index, "Results", reports 80% to 93% for a text's own hot third)."""
    order = np.argsort(uniform_u64(base, "hot.set", E), kind="stable")
    hot = order[: int(round(E * hot_frac))]
    b = np.zeros(E, dtype=np.float64)
    b[hot] = bias
    return b, np.sort(hot)
