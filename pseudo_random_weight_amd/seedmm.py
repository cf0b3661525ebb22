"""Thin Python binding of the seedmm C ABI (include/seedmm.h).

Argument marshalling only: tensors are passed to the HIP library as device pointers
plus sizes, on torch's current HIP stream or the one passed in (outputs and scratch the
binding allocates belong to that stream).  Every step of the computation runs in
the library's kernels; there is no Python or CPU fallback, and a missing library
raises at import.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libseedmm.so")

OK, EINVAL, EALIGN, EWORKSPACE, EHIP, ECAPACITY, ESCRATCH = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 8 << 20      # SEEDMM_NOALLOC_SCRATCH_BYTES of include/seedmm.h


class SeedmmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_lib.seedmm_strerror(status).decode()} (status {status})")
        self.status = status


class SeedMat(ctypes.Structure):
    _fields_ = [("seeds", ctypes.c_void_p), ("coefs", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("exp_bias", ctypes.c_void_p)]


class SeedSide(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("fork", ctypes.c_void_p),
                ("join", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m pseudo_random_weight_amd.build` "
            "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    p, i32 = ctypes.c_void_p, ctypes.c_int
    L.seedmm_gemv.argtypes = [p, p, p, ctypes.c_int32, p, p, i32, i32, i32]
    L.seedmm_gemv_ex.argtypes = [p, p, p, ctypes.c_int32, p, i32, i32, p, i32, i32, i32, i32, i32, p]
    L.seedmm_reconstruct.argtypes = [p, p, p, ctypes.c_int32, p, i32, i32, i32, i32, p]
    L.seedmm_moe_dispatch.argtypes = [p, i32, i32, i32, p, p, p]
    L.seedmm_moe_workspace_bytes.restype = ctypes.c_size_t
    L.seedmm_moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.seedmm_moe.argtypes = [p, p, i32, i32, p, p, i32, i32, i32, i32, SeedMat, SeedMat, SeedMat,
                             p, ctypes.c_size_t, p]
    L.seedmm_moe_timed.argtypes = L.seedmm_moe.argtypes + [p]
    L.seedmm_moe_noalloc.argtypes = [p, p, i32, i32, p, p, i32, i32, i32, i32, SeedMat, SeedMat,
                                     SeedMat, p]
    L.seedmm_moe_ex.argtypes = [p, p, i32, i32, p, p, i32, i32, i32, i32, p, SeedMat, SeedMat,
                                SeedMat, p, ctypes.c_size_t, p, ctypes.POINTER(SeedSide)]
    L.seedmm_search.argtypes = [p, i32, p, i32, i32, i32, ctypes.c_int32, p, p, p, p, p, p]
    L.seedmm_search_table_bytes.restype = ctypes.c_size_t
    L.seedmm_search_table_bytes.argtypes = [i32]
    L.seedmm_search_prepare.argtypes = [i32, p, ctypes.c_size_t, p]
    L.seedmm_moe_mixed.argtypes = [p, p, i32, i32, p, p, i32, i32, i32, p, SeedMat, SeedMat,
                                   SeedMat, p, ctypes.c_size_t, p]
    sz = ctypes.c_size_t
    L.seedmm_cache_state_bytes.restype = sz
    L.seedmm_cache_state_bytes.argtypes = [i32, i32]
    L.seedmm_cache_device_bytes.restype = sz
    L.seedmm_cache_device_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.seedmm_cache_record_layout.restype = sz
    L.seedmm_cache_record_layout.argtypes = [i32, i32, i32, p]
    L.seedmm_cache_init.argtypes = [p, sz, i32, i32, i32, i32, i32, p, p, p, sz]
    L.seedmm_cache_reset.argtypes = [p]
    L.seedmm_cache_plan.argtypes = [p, p, i32, i32, p, p]
    L.seedmm_cache_moe.argtypes = [p, p, p, p, i32, i32, p, p, p, sz, p]
    L.seedmm_cache_stats.argtypes = [p, p]
    L.seedmm_strerror.restype = ctypes.c_char_p
    L.seedmm_strerror.argtypes = [i32]
    L.seedmm_version.restype = i32
    for name in ("seedmm_gemv", "seedmm_gemv_ex", "seedmm_reconstruct", "seedmm_moe_dispatch",
                 "seedmm_moe", "seedmm_moe_timed", "seedmm_moe_ex", "seedmm_moe_noalloc",
                 "seedmm_search",
                 "seedmm_search_prepare", "seedmm_moe_mixed",
                 "seedmm_cache_init", "seedmm_cache_reset", "seedmm_cache_plan",
                 "seedmm_cache_moe", "seedmm_cache_stats"):
        getattr(L, name).restype = i32
    return L


_lib = _load()

EXPORTS = ("seedmm_gemv", "seedmm_gemv_ex", "seedmm_reconstruct", "seedmm_moe_dispatch",
           "seedmm_moe_workspace_bytes", "seedmm_moe", "seedmm_moe_timed", "seedmm_moe_ex",
           "seedmm_moe_noalloc",
           "seedmm_moe_mixed", "seedmm_search", "seedmm_search_table_bytes",
           "seedmm_search_prepare", "seedmm_cache_record_layout", "seedmm_cache_state_bytes",
           "seedmm_cache_device_bytes",
           "seedmm_cache_init", "seedmm_cache_reset", "seedmm_cache_plan", "seedmm_cache_moe",
           "seedmm_cache_stats", "seedmm_strerror", "seedmm_version")


def lib():
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


# raw handle of a device's current stream without building a torch Stream object
_raw_current = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream_handle(index=None) -> int:
    if index is None:
        index = torch.cuda.current_device()
    if _raw_current is not None:
        return _raw_current(index)
    return torch.cuda.current_stream(index).cuda_stream


def _stream(stream=None):
    if stream is None:
        return ctypes.c_void_p(_current_stream_handle())
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Allocation context: new tensors belong to `stream` (None: the current stream), so
    the caching allocator does not hand their memory to other streams while the
    library's kernels on `stream` may still use it."""
    return torch.cuda.stream(stream) if stream is not None else _Nothing()


class _Nothing:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


class SideStream:
    """A second stream of one device and its fork / join events, for moe(side=...) and
    moe_mixed(side=...): the layer runs one half of its expert launches there
    (seedmm_moe_ex).  Owned by the caller; concurrent layer calls need one each."""

    def __init__(self, device=None):
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.stream = torch.cuda.Stream(device=dev)          # default priority
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()
        # torch creates an event on its first record: record both once so handles exist
        self.fork.record(self.stream)
        self.join.record(self.stream)
        self.stream.synchronize()

    def c(self) -> SeedSide:
        return SeedSide(self.stream.cuda_stream, self.fork.cuda_event, self.join.cuda_event)


def _check(status: int, what: str):
    if status != OK:
        raise SeedmmError(status, what)


def _dev(t, dtype, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _mat(m: dict):
    _dev(m["seeds"], torch.uint16, "seeds")
    _dev(m["coefs"], torch.uint16, "coefs")
    _dev(m["codes"], torch.uint8, "codes")
    return m


def stream_sizes(E: int, M: int, K: int, Ps) -> dict:
    """Elements of the seeds (u16), coefs (u16) and codes (u8) streams of E stacked [M][K]
    matrices; Ps is one P for all, or a P per matrix (mixed packs)."""
    n = M * (K // 8)
    Ps = [int(Ps)] * E if isinstance(Ps, int) else [int(p) for p in Ps]
    if len(Ps) != E:
        raise ValueError(f"{len(Ps)} values of P for {E} matrices")
    coef_nibbles = sum(n * p for p in Ps)
    return {"seeds": E * n, "coefs": (coef_nibbles + 3) // 4, "codes": (E * n + 1) // 2}


def _check_streams(m: dict, E: int, M: int, K: int, Ps, name: str, exact_coefs=True):
    """The kernels index the streams from (E, M, K, P) alone: a stream shorter than that
    would be read out of bounds, so it is refused here, before anything is launched."""
    need = stream_sizes(E, M, K, Ps)
    for k, n in need.items():
        if not exact_coefs and k == "coefs":
            continue
        if m[k].numel() < n:
            raise ValueError(f"{name}.{k} has {m[k].numel()} elements; {E} stacked {M}x{K} "
                             f"matrices need {n}")
    eb = m.get("exp_bias")
    if isinstance(eb, torch.Tensor) and eb.numel() < E:
        raise ValueError(f"{name}.exp_bias has {eb.numel()} entries for {E} matrices")


def _check_numel(t, n, name):
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, {n} needed")


def gemv(mat: dict, x: torch.Tensor, M: int, K: int, P: int, y: torch.Tensor = None):
    """y = W x for fp32 x[K] (seedmm_gemv).  The C call has no stream argument and runs on
    the null stream; under another current stream the binding orders it after that
    stream's earlier work and that stream's later work after it (events, no host wait)."""
    _mat(mat)
    _check_streams(mat, 1, M, K, P, "W")
    _dev(x, torch.float32, "x")
    _check_numel(x, K, "x")
    if y is None:
        y = torch.empty(M, dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, "y")
    _check_numel(y, M, "y")
    eb = int(mat["exp_bias_host"][0]) if "exp_bias_host" in mat else int(mat["exp_bias"][0])
    args = (_ptr(mat["seeds"]), _ptr(mat["coefs"]), _ptr(mat["codes"]), eb, _ptr(x), _ptr(y),
            M, K, P)
    idx = x.device.index
    if idx == torch.cuda.current_device() and _current_stream_handle(idx) == 0:
        status = _lib.seedmm_gemv(*args)       # torch's default stream is the null stream
    else:
        with torch.cuda.device(x.device):
            cur, null = torch.cuda.current_stream(), torch.cuda.default_stream()
            null.wait_stream(cur)
            status = _lib.seedmm_gemv(*args)
            cur.wait_stream(null)
    _check(status, "seedmm_gemv")
    return y


def gemv_ex(mat: dict, x: torch.Tensor, M: int, K: int, P: int, y: torch.Tensor = None,
            stream=None):
    """Y[n] = W X[n] for X fp32 or bf16 [N][K] (seedmm_gemv_ex)."""
    _mat(mat)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _dev(x, x.dtype, "x")
    _check_streams(mat, 1, M, K, P, "W")
    N = x.shape[0] if x.dim() == 2 else 1
    ldx = x.shape[-1]
    if ldx < K:
        raise ValueError(f"x rows hold {ldx} elements, K = {K}")
    if y is None:
        with _on(stream):
            y = torch.empty((N, M), dtype=torch.float32, device=x.device)
    _dev(y, torch.float32, "y")
    if y.shape[-1] < M or y.numel() < N * y.shape[-1]:
        raise ValueError(f"y must hold [{N}][{M}]")
    eb = int(mat["exp_bias_host"][0]) if "exp_bias_host" in mat else int(mat["exp_bias"][0])
    _check(_lib.seedmm_gemv_ex(_ptr(mat["seeds"]), _ptr(mat["coefs"]), _ptr(mat["codes"]), eb,
                               _ptr(x), F32 if x.dtype == torch.float32 else BF16, ldx, _ptr(y),
                               y.shape[-1], M, K, P, N, _stream(stream)), "seedmm_gemv_ex")
    return y


def reconstruct(mat: dict, M: int, K: int, P: int, dtype=torch.float32, out=None, stream=None):
    """W[M][K] in fp32 (exact) or bf16 (seedmm_reconstruct)."""
    _mat(mat)
    _check_streams(mat, 1, M, K, P, "W")
    dev = mat["seeds"].device
    if out is None:
        with _on(stream):
            out = torch.empty((M, K), dtype=dtype, device=dev)
    _dev(out, dtype, "W")
    _check_numel(out, M * K, "W")
    eb = int(mat["exp_bias_host"][0]) if "exp_bias_host" in mat else int(mat["exp_bias"][0])
    _check(_lib.seedmm_reconstruct(_ptr(mat["seeds"]), _ptr(mat["coefs"]), _ptr(mat["codes"]), eb,
                                   _ptr(out), F32 if dtype == torch.float32 else BF16, M, K, P,
                                   _stream(stream)), "seedmm_reconstruct")
    return out


def moe_dispatch(topk_ids: torch.Tensor, E: int, stream=None):
    """(counts int32[E], lists int32[E][T]) for topk_ids int32 [T][top_k]."""
    _dev(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    with _on(stream):
        counts = torch.empty(E, dtype=torch.int32, device=topk_ids.device)
        lists = torch.full((E, max(T, 1)), -1, dtype=torch.int32, device=topk_ids.device)
    _check(_lib.seedmm_moe_dispatch(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(lists),
                                    _stream(stream)), "seedmm_moe_dispatch")
    return counts, lists


def moe_workspace_bytes(T: int, top_k: int, E: int, H: int, I: int) -> int:
    return int(_lib.seedmm_moe_workspace_bytes(T, top_k, E, H, I))


def _seedmat(m: dict) -> SeedMat:
    _mat(m)
    _dev(m["exp_bias"], torch.int32, "exp_bias")
    return SeedMat(m["seeds"].data_ptr(), m["coefs"].data_ptr(), m["codes"].data_ptr(),
                   m["exp_bias"].data_ptr())


def _check_layer(T, k, topk_w, x, E, H, I, Ps, gate, up, down, exact_coefs=True):
    _check_numel(topk_w, T * k, "topk_w")
    _check_numel(x, T * H, "x")
    for name, m, (M, K) in (("gate", gate, (I, H)), ("up", up, (I, H)), ("down", down, (H, I))):
        _check_streams(m, E, M, K, Ps, name, exact_coefs)


def check_topk_ids(topk_ids, E: int):
    """Host check of a routing's expert ids, which the layer calls leave to the caller:
    every id in [0, E) and the top_k ids of each token distinct.  Copies the ids to the
    host (a synchronisation); raises ValueError naming the first token that breaks it."""
    ids = topk_ids.detach().to("cpu").to(torch.int64)
    if ids.dim() != 2:
        raise ValueError("topk_ids must be [T][top_k]")
    bad = ((ids < 0) | (ids >= E)).any(dim=1)
    if bool(bad.any()):
        t = int(bad.nonzero()[0, 0])
        raise ValueError(f"topk_ids[{t}] holds an expert id outside [0, {E})")
    if ids.shape[1] > 1:
        srt = ids.sort(dim=1).values
        dup = (srt[:, 1:] == srt[:, :-1]).any(dim=1)
        if bool(dup.any()):
            t = int(dup.nonzero()[0, 0])
            raise ValueError(f"topk_ids[{t}] names one expert twice")


def moe(topk_ids, topk_w, x, E, H, I, P, gate, up, down, y=None, workspace=None, stream=None,
        events=None, side=None, check_ids=False):
    """Routed SwiGLU MoE layer (seedmm_moe); x bf16 [T][H] -> y fp32 [T][H].
    `events`: optional 5 raw hipEvent_t handles (ints) recorded between the stages
    (seedmm_moe_timed).  `side`: optional SideStream for the second half of the expert
    launches (seedmm_moe_ex).  `check_ids`: validate topk_ids on the host first
    (check_topk_ids)."""
    if check_ids:
        check_topk_ids(topk_ids, E)
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(topk_w, torch.float32, "topk_w")
    _dev(x, torch.bfloat16, "x")
    T, k = topk_ids.shape
    _check_layer(T, k, topk_w, x, E, H, I, P, gate, up, down)
    if events is not None and side is not None:
        raise ValueError("the timed layer call runs on one stream (no side stream)")
    with _on(stream):
        if y is None:
            y = torch.empty((T, H), dtype=torch.float32, device=x.device)
        need = moe_workspace_bytes(T, k, E, H, I)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _dev(y, torch.float32, "y")
    _check_numel(y, T * H, "y")
    args = (_ptr(topk_ids), _ptr(topk_w), T, k, _ptr(x), _ptr(y), E, H, I, P,
            _seedmat(gate), _seedmat(up), _seedmat(down), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if events is not None:
        arr = (ctypes.c_void_p * 5)(*[getattr(ev, "cuda_event", ev) for ev in events])
        _check(_lib.seedmm_moe_timed(*args, arr), "seedmm_moe_timed")
    elif side is not None:
        sd = side.c()
        _check(_lib.seedmm_moe_ex(*args[:10], None, *args[10:], ctypes.byref(sd)),
               "seedmm_moe_ex")
    else:
        _check(_lib.seedmm_moe(*args), "seedmm_moe")
    return y


def p4_mask(Ps, device) -> torch.Tensor:
    """Device bitmask of the experts with P = 4 (bit e of word e // 32)."""
    E = len(Ps)
    words = [0] * ((E + 31) // 32)
    for e, P in enumerate(Ps):
        if int(P) == 4:
            words[e >> 5] |= 1 << (e & 31)
        elif int(P) != 3:
            raise ValueError("every expert's P must be 3 or 4")
    return torch.tensor([w - (1 << 32) if w >= (1 << 31) else w for w in words],
                        dtype=torch.int32, device=device)


def moe_mixed(topk_ids, topk_w, x, E, H, I, p4mask, gate, up, down, y=None, workspace=None,
              stream=None, Ps=None, side=None, check_ids=False):
    """Routed SwiGLU MoE layer with P chosen per expert (seedmm_moe_mixed); p4mask from
    p4_mask(Ps).  Given Ps, the coefficient streams are checked against it; without, only
    the seed and code streams are (the mask lives on the device).  `side`: optional
    SideStream for the P = 3 launches (seedmm_moe_ex with P = 0).  `check_ids`: validate
    topk_ids on the host first (check_topk_ids)."""
    if check_ids:
        check_topk_ids(topk_ids, E)
    _dev(topk_ids, torch.int32, "topk_ids")
    _dev(topk_w, torch.float32, "topk_w")
    _dev(x, torch.bfloat16, "x")
    _dev(p4mask, torch.int32, "p4mask")
    _check_numel(p4mask, (E + 31) // 32, "p4mask")
    T, k = topk_ids.shape
    _check_layer(T, k, topk_w, x, E, H, I, Ps if Ps is not None else 3, gate, up, down,
                 exact_coefs=Ps is not None)
    with _on(stream):
        if y is None:
            y = torch.empty((T, H), dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = torch.empty(moe_workspace_bytes(T, k, E, H, I), dtype=torch.uint8,
                                    device=x.device)
    _dev(y, torch.float32, "y")
    _check_numel(y, T * H, "y")
    args = (_ptr(topk_ids), _ptr(topk_w), T, k, _ptr(x), _ptr(y), E, H, I)
    rest = (_seedmat(gate), _seedmat(up), _seedmat(down), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if side is not None:
        sd = side.c()
        _check(_lib.seedmm_moe_ex(*args, 0, _ptr(p4mask), *rest, ctypes.byref(sd)),
               "seedmm_moe_ex")
    else:
        _check(_lib.seedmm_moe_mixed(*args, _ptr(p4mask), *rest), "seedmm_moe_mixed")
    return y


_TABLES = {}


def search_table(P: int, device=None, stream=None):
    """The encoder's per-seed table for P on a device (seedmm_search_prepare), filled
    once and kept by this module for later searches on that device."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    key = (dev.index, int(P))
    if key not in _TABLES:
        n = int(_lib.seedmm_search_table_bytes(P))
        if n == 0:
            raise SeedmmError(EINVAL, "seedmm_search_table_bytes")
        with torch.cuda.device(dev):   # the fill runs on that device (its current stream if none given)
            with _on(stream):
                buf = torch.empty(n + 256, dtype=torch.uint8, device=dev)
            off = (-buf.data_ptr()) % 256
            tab = buf[off:off + n]
            _check(_lib.seedmm_search_prepare(P, _ptr(tab), n, _stream(stream)),
                   "seedmm_search_prepare")
            # later searches may run on other streams: wait for the fill once, here
            (stream or torch.cuda.current_stream()).synchronize()
        _TABLES[key] = (buf, tab)
    return _TABLES[key][1]


def search(W: torch.Tensor, P: int, exp_bias: int, colw: torch.Tensor = None, err=True,
           stream=None):
    """Encode fp32 W [M][K] by the exhaustive seed search (seedmm_search): a dict with
    seeds, coefs, codes (device tensors, the products' layout), exp_bias and, if asked,
    err (float64 [M*K/8], squared error of every block)."""
    _dev(W, torch.float32, "W")
    M, K = W.shape
    if colw is not None:
        _dev(colw, torch.float32, "colw")
        _check_numel(colw, K, "colw")
    nblk = M * (K // 8)
    dev = W.device
    table = search_table(P, dev, stream) if colw is None else None
    with _on(stream):
        out = {"seeds": torch.empty(nblk, dtype=torch.uint16, device=dev),
               "coefs": torch.empty((nblk * P + 3) // 4, dtype=torch.uint16, device=dev),
               "codes": torch.empty((nblk + 1) // 2, dtype=torch.uint8, device=dev),
               "exp_bias": torch.full((1,), exp_bias, dtype=torch.int32, device=dev),
               "exp_bias_host": [exp_bias]}
        e = torch.empty(nblk, dtype=torch.float64, device=dev) if err else None
    _check(_lib.seedmm_search(_ptr(W), K, _ptr(colw), M, K, P, exp_bias, _ptr(out["seeds"]),
                              _ptr(out["coefs"]), _ptr(out["codes"]), _ptr(e), _ptr(table),
                              _stream(stream)), "seedmm_search")
    if err:
        out["err"] = e
    return out


class ExpertCache:
    """A layer whose routed experts live in pinned host memory, with S device slots for
    the recently used ones (seedmm_cache_*).  Calls must reach the device in call order:
    use one stream for every call on a cache (a call's record copies can overwrite slots
    the previous call still reads).  host: {"gate", "up", "down"} -> dicts of
    numpy streams (seeds, coefs, codes, exp_bias) stacked as for moe(); they are packed
    once into expert records in pinned host memory (offsets from
    seedmm_cache_record_layout), and the exp_bias arrays go to device memory."""

    def __init__(self, host: dict, E: int, H: int, I: int, P: int, S: int, device="cuda"):
        import numpy as np
        self.E, self.H, self.I, self.P, self.S = E, H, I, P, S
        offs = (ctypes.c_size_t * 9)()
        rec = int(_lib.seedmm_cache_record_layout(H, I, P, offs))
        nstate = int(_lib.seedmm_cache_state_bytes(E, S))
        ndev = int(_lib.seedmm_cache_device_bytes(E, H, I, P, S))
        if rec == 0 or nstate == 0 or ndev == 0:
            raise SeedmmError(EINVAL, "seedmm_cache sizes")
        self.record_bytes = rec
        for n, (M, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            need = stream_sizes(E, M, K, P)
            for part, cnt in need.items():
                if np.asarray(host[n][part]).size < cnt:
                    raise ValueError(f"{n}.{part} has {np.asarray(host[n][part]).size} "
                                     f"elements; {E} stacked {M}x{K} matrices need {cnt}")
            if np.asarray(host[n]["exp_bias"]).size < E:
                raise ValueError(f"{n}.exp_bias has fewer than {E} entries")
        pack = torch.zeros(E * rec, dtype=torch.uint8, pin_memory=True)
        view = pack.numpy().reshape(E, rec)
        for m, n in enumerate(("gate", "up", "down")):
            for k, part in enumerate(("seeds", "coefs", "codes")):
                a = np.ascontiguousarray(host[n][part]).view(np.uint8).reshape(E, -1)
                o = offs[3 * m + k]
                view[:, o:o + a.shape[1]] = a
        self._pack = pack
        eb = np.stack([np.asarray(host[n]["exp_bias"], dtype=np.int32) for n in ("gate", "up", "down")])
        self._exp_bias = torch.from_numpy(np.ascontiguousarray(eb)).to(device)
        self._state = torch.empty((nstate + 7) // 8, dtype=torch.int64)   # host, 8-byte aligned
        self._device = torch.empty(ndev + 256, dtype=torch.uint8, device=device)
        off = (-self._device.data_ptr()) % 256
        _check(_lib.seedmm_cache_init(self.handle, nstate, E, H, I, P, S,
                                      ctypes.c_void_p(pack.data_ptr()),
                                      ctypes.c_void_p(self._exp_bias.data_ptr()),
                                      ctypes.c_void_p(self._device.data_ptr() + off), ndev),
               "seedmm_cache_init")

    @property
    def handle(self):
        return ctypes.c_void_p(self._state.data_ptr())

    @property
    def device_bytes(self) -> int:
        return int(_lib.seedmm_cache_device_bytes(self.E, self.H, self.I, self.P, self.S))

    def reset(self):
        _check(_lib.seedmm_cache_reset(self.handle), "seedmm_cache_reset")

    def plan(self, topk_ids_host):
        """Host-only plan of one call: [(expert, slot), ...] loads (changes the state)."""
        import numpy as np
        ids = np.ascontiguousarray(topk_ids_host, dtype=np.int32)
        T, k = ids.shape
        loads = np.zeros(2 * self.S, dtype=np.int32)
        n = ctypes.c_int(0)
        _check(_lib.seedmm_cache_plan(self.handle, ids.ctypes.data_as(ctypes.c_void_p), T, k,
                                      loads.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)),
               "seedmm_cache_plan")
        return [(int(loads[2 * i]), int(loads[2 * i + 1])) for i in range(n.value)]

    def moe(self, topk_ids_host, topk_ids, topk_w, x, y=None, workspace=None, stream=None):
        """The routed layer through the cache (seedmm_cache_moe); topk_ids_host is the
        host copy (numpy int32 [T][top_k]) of the device topk_ids."""
        import numpy as np
        ids_h = np.ascontiguousarray(topk_ids_host, dtype=np.int32)
        _dev(topk_ids, torch.int32, "topk_ids")
        _dev(topk_w, torch.float32, "topk_w")
        _dev(x, torch.bfloat16, "x")
        T, k = topk_ids.shape
        if ids_h.shape != (T, k):
            raise ValueError("topk_ids_host and topk_ids differ in shape")
        _check_numel(topk_w, T * k, "topk_w")
        _check_numel(x, T * self.H, "x")
        with _on(stream):
            if y is None:
                y = torch.empty((T, self.H), dtype=torch.float32, device=x.device)
            if workspace is None:
                workspace = torch.empty(moe_workspace_bytes(T, k, self.E, self.H, self.I),
                                        dtype=torch.uint8, device=x.device)
        _dev(y, torch.float32, "y")
        _check_numel(y, T * self.H, "y")
        _check(_lib.seedmm_cache_moe(self.handle, ids_h.ctypes.data_as(ctypes.c_void_p),
                                     _ptr(topk_ids), _ptr(topk_w), T, k, _ptr(x), _ptr(y),
                                     _ptr(workspace),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream)), "seedmm_cache_moe")
        return y

    def stats(self) -> dict:
        out = (ctypes.c_uint64 * 5)()
        _check(_lib.seedmm_cache_stats(self.handle, out), "seedmm_cache_stats")
        return dict(zip(("calls", "uses", "hits", "misses", "bytes"), (int(v) for v in out)))
