"""ctypes wrapper over the C oracle (oracle/seedref.c).

TEST INFRASTRUCTURE ONLY.  Imported by tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg; the GPU library and its binding never import it.
It shares no code with the HIP path.  All arrays are host numpy arrays.

Parity status: pinned by the CPU tests (tests/test_oracle_*.py) against the pages'
closed forms and invariants, exhaustive checks, brute force and library reductions.
Parity unpinned: the tap mask and the basis fill order are readings of the pages, and
bit-compatibility with the published model files cannot be checked (the pages print
no worked example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libseedref.so")
_SRC = os.path.join(_HERE, "seedref.c")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-ffp-contract=off keeps every product and sum
    separately rounded, as the C reference of the pages requires)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-ffp-contract=off", "-fopenmp",
               "-shared", "-fPIC", _SRC, "-o", _SO + ".tmp", "-lm"]
        subprocess.check_call(cmd, cwd=_HERE)
        os.replace(_SO + ".tmp", _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        p = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.seedref_lfsr_step.restype = ctypes.c_uint16
        L.seedref_lfsr_step.argtypes = [ctypes.c_uint16]
        L.seedref_states.argtypes = [ctypes.c_uint16, i32, p]
        L.seedref_coef.argtypes = [p, i64, i32, i32]
        L.seedref_code.argtypes = [p, i64]
        L.seedref_block.argtypes = [ctypes.c_uint16, p, i32, i32, i32, p]
        L.seedref_stream_bytes.argtypes = [i64, i64, i32, p, p, p]
        L.seedref_reconstruct_f32.argtypes = [p, p, p, i32, i32, i32, i32, p]
        L.seedref_reconstruct_bf16.argtypes = [p, p, p, i32, i32, i32, i32, p]
        L.seedref_f32_to_bf16.restype = ctypes.c_uint16
        L.seedref_f32_to_bf16.argtypes = [ctypes.c_float]
        L.seedref_gemv.argtypes = [p, p, p, i32, p, i32, p, i32, i32, i32, i32, i32]
        L.seedref_expert_accum.argtypes = [p, p, p, i32, p, p, p, i32, p, p, p, i32,
                                           p, f64, p, i32, i32, i32]
        L.seedref_moe.argtypes = [p, p, i32, i32, p, p, i32, i32, i32, i32] + [p] * 12
        L.seedref_moe_mixed.argtypes = [p, p, i32, i32, p, p, i32, i32, i32, p] + [p] * 12
        L.seedref_search_block.argtypes = [p, i32, i32, p, p, p, p]
        L.seedref_search_block_w.argtypes = [p, p, i32, i32, p, p, p, p]
        L.seedref_search_matrix.argtypes = [p, p, i32, i32, i32, i32, p, p, p, p]
        L.seedref_num_threads.restype = ctypes.c_int
        L.seedref_set_num_threads.restype = None
        L.seedref_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {rc})")


def lfsr_step(s: int) -> int:
    return int(lib().seedref_lfsr_step(s))


def states(seed: int, n: int) -> np.ndarray:
    out = np.zeros(n, dtype=np.uint16)
    lib().seedref_states(seed, n, _ptr(out))
    return out


def coef(coefs: np.ndarray, b: int, P: int, j: int) -> int:
    return int(lib().seedref_coef(_ptr(coefs), b, P, j))


def code(codes: np.ndarray, b: int) -> int:
    return int(lib().seedref_code(_ptr(codes), b))


def block(seed: int, c, P: int, code_: int, exp_bias: int) -> np.ndarray:
    ca = np.zeros(4, dtype=np.int32)
    ca[:P] = c[:P]
    w = np.zeros(8, dtype=np.float32)
    lib().seedref_block(seed, _ptr(ca), P, code_, exp_bias, _ptr(w))
    return w


def stream_bytes(M: int, K: int, P: int):
    a, b, c = (np.zeros(1, dtype=np.int64) for _ in range(3))
    _check(lib().seedref_stream_bytes(M, K, P, _ptr(a), _ptr(b), _ptr(c)), "stream_bytes")
    return int(a[0]), int(b[0]), int(c[0])


def reconstruct_f32(mat: dict, M: int, K: int, P: int, e: int = 0) -> np.ndarray:
    s, c, d, eb = _expert_view(mat, M, K, P, e)
    W = np.zeros((M, K), dtype=np.float32)
    _check(lib().seedref_reconstruct_f32(_ptr(s), _ptr(c), _ptr(d), int(eb), M, K, P, _ptr(W)),
           "reconstruct_f32")
    return W


def reconstruct_bf16(mat: dict, M: int, K: int, P: int, e: int = 0) -> np.ndarray:
    s, c, d, eb = _expert_view(mat, M, K, P, e)
    W = np.zeros((M, K), dtype=np.uint16)
    _check(lib().seedref_reconstruct_bf16(_ptr(s), _ptr(c), _ptr(d), int(eb), M, K, P, _ptr(W)),
           "reconstruct_bf16")
    return W


def f32_to_bf16(f: float) -> int:
    return int(lib().seedref_f32_to_bf16(f))


def gemv(mat: dict, x: np.ndarray, M: int, K: int, P: int, e: int = 0) -> np.ndarray:
    """y[n][m] for x fp32 [N][K] (double accumulation)."""
    s, c, d, eb = _expert_view(mat, M, K, P, e)
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, K)
    N = x.shape[0]
    y = np.zeros((N, M), dtype=np.float32)
    _check(lib().seedref_gemv(_ptr(s), _ptr(c), _ptr(d), int(eb), _ptr(x), K, _ptr(y), M,
                              M, K, P, N), "gemv")
    return y


def _expert_view(mat: dict, M: int, K: int, P: int, e: int):
    """Streams of expert e of a stacked tensor (whole words/bytes per expert)."""
    nblk = M * (K // 8)
    if e == 0:
        return (np.ascontiguousarray(mat["seeds"]), np.ascontiguousarray(mat["coefs"]),
                np.ascontiguousarray(mat["codes"]), int(mat["exp_bias"][0]))
    assert (nblk * P) % 4 == 0 and nblk % 2 == 0
    cw, cb = nblk * P // 4, nblk // 2
    return (np.ascontiguousarray(mat["seeds"][e * nblk:(e + 1) * nblk]),
            np.ascontiguousarray(mat["coefs"][e * cw:(e + 1) * cw]),
            np.ascontiguousarray(mat["codes"][e * cb:(e + 1) * cb]),
            int(mat["exp_bias"][e]))


def expert(gate: dict, up: dict, down: dict, x: np.ndarray, H: int, I: int, P: int,
           e: int = 0) -> np.ndarray:
    """One SwiGLU expert on x fp32 [T][H] -> float64 [T][H]."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, H)
    g = _expert_view(gate, I, H, P, e)
    u = _expert_view(up, I, H, P, e)
    d = _expert_view(down, H, I, P, e)
    out = np.zeros((x.shape[0], H), dtype=np.float64)
    for t in range(x.shape[0]):
        xt = np.ascontiguousarray(x[t])
        yt = np.zeros(H, dtype=np.float64)
        _check(lib().seedref_expert_accum(
            _ptr(g[0]), _ptr(g[1]), _ptr(g[2]), g[3], _ptr(u[0]), _ptr(u[1]), _ptr(u[2]), u[3],
            _ptr(d[0]), _ptr(d[1]), _ptr(d[2]), d[3], _ptr(xt), 1.0, _ptr(yt), H, I, P), "expert")
        out[t] = yt
    return out


def moe(topk_ids: np.ndarray, topk_w: np.ndarray, x: np.ndarray, E: int, H: int, I: int, P: int,
        gate: dict, up: dict, down: dict) -> np.ndarray:
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, k = ids.shape
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(T, H)
    y = np.zeros((T, H), dtype=np.float32)
    args = []
    for m in (gate, up, down):
        args += [_ptr(np.ascontiguousarray(m["seeds"])), _ptr(np.ascontiguousarray(m["coefs"])),
                 _ptr(np.ascontiguousarray(m["codes"])),
                 _ptr(np.ascontiguousarray(m["exp_bias"], dtype=np.int32))]
    _check(lib().seedref_moe(_ptr(ids), _ptr(w), T, k, _ptr(x), _ptr(y), E, H, I, P, *args), "moe")
    return y


def moe_mixed(topk_ids: np.ndarray, topk_w: np.ndarray, x: np.ndarray, E: int, H: int, I: int,
              Pe, gate: dict, up: dict, down: dict) -> np.ndarray:
    """The routed layer with P chosen per expert (Pe: E values, 3 or 4)."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, k = ids.shape
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(T, H)
    y = np.zeros((T, H), dtype=np.float32)
    pe = np.ascontiguousarray(Pe, dtype=np.int32)
    args = []
    for m in (gate, up, down):
        args += [_ptr(np.ascontiguousarray(m["seeds"])), _ptr(np.ascontiguousarray(m["coefs"])),
                 _ptr(np.ascontiguousarray(m["codes"])),
                 _ptr(np.ascontiguousarray(m["exp_bias"], dtype=np.int32))]
    _check(lib().seedref_moe_mixed(_ptr(ids), _ptr(w), T, k, _ptr(x), _ptr(y), E, H, I, _ptr(pe),
                                   *args), "moe_mixed")
    return y


def search_block(w8: np.ndarray, exp_bias: int, P: int, d8: np.ndarray = None):
    """(seed, coefficients, code, squared error) of the exhaustive search for one block;
    d8: importance of each of the 8 weights (None: unweighted)."""
    w = np.ascontiguousarray(w8, dtype=np.float64)
    seed = np.zeros(1, dtype=np.uint16)
    c = np.zeros(4, dtype=np.int32)
    cd = np.zeros(1, dtype=np.int32)
    err = np.zeros(1, dtype=np.float64)
    if d8 is None:
        rc = lib().seedref_search_block(_ptr(w), exp_bias, P, _ptr(seed), _ptr(c), _ptr(cd),
                                        _ptr(err))
    else:
        d = np.ascontiguousarray(d8, dtype=np.float64)
        rc = lib().seedref_search_block_w(_ptr(w), _ptr(d), exp_bias, P, _ptr(seed), _ptr(c),
                                          _ptr(cd), _ptr(err))
    _check(rc, "search_block")
    return int(seed[0]), [int(v) for v in c[:P]], int(cd[0]), float(err[0])


def search_matrix(W: np.ndarray, P: int, exp_bias: int, colw: np.ndarray = None):
    """Encode fp32 W [M][K] block by block: a seed-coded matrix dict (seeds, coefs,
    codes, exp_bias) plus the squared error of every block ('err', float64 [M*K/8])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    M, K = W.shape
    nblk = M * (K // 8)
    seeds = np.zeros(nblk, dtype=np.uint16)
    coefs = np.zeros((nblk * P + 3) // 4, dtype=np.uint16)
    codes = np.zeros((nblk + 1) // 2, dtype=np.uint8)
    err = np.zeros(nblk, dtype=np.float64)
    cw = None if colw is None else np.ascontiguousarray(colw, dtype=np.float32)
    _check(lib().seedref_search_matrix(_ptr(W), None if cw is None else _ptr(cw), M, K, P,
                                       exp_bias, _ptr(seeds), _ptr(coefs), _ptr(codes),
                                       _ptr(err)), "search_matrix")
    return {"seeds": seeds, "coefs": coefs, "codes": codes,
            "exp_bias": np.array([exp_bias], dtype=np.int32), "err": err}


def num_threads() -> int:
    return int(lib().seedref_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's parallel loops (results do not depend on it)."""
    lib().seedref_set_num_threads(int(n))
