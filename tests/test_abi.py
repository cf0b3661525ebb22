"""CPU checks of the C-ABI library: it loads, exports every declared symbol, and
rejects bad arguments before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seedmm.h")
SO = os.path.join(ROOT, "pseudo_random_weight_amd", "libseedmm.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(seedmm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(SO):
        pytest.fail("libseedmm.so is not built (python -m pseudo_random_weight_amd.build)")
    from pseudo_random_weight_amd import seedmm
    return seedmm.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    from pseudo_random_weight_amd import seedmm
    assert set(seedmm.EXPORTS) == set(names)


def test_version_and_strerror(lib):
    assert lib.seedmm_version() >= 100
    for st in (0, -1, -2, -3, -4, 7):
        assert isinstance(lib.seedmm_strerror(st), bytes)


FAKE = 0x100000   # 16-byte aligned address that is never dereferenced: validation fails first


@pytest.mark.parametrize("M,K,P,eb,expect", [
    (16, 12, 4, 0, -1),      # K % 8
    (16, 16, 5, 0, -1),      # P
    (16, 16, 2, 0, -1),
    (-1, 16, 4, 0, -1),      # M < 0
    (16, 16, 4, 101, -1),    # exp_bias out of range
    (16, 16, 4, -101, -1),
])
def test_gemv_rejects_bad_shapes(lib, M, K, P, eb, expect):
    assert lib.seedmm_gemv(FAKE, FAKE, FAKE, eb, FAKE, FAKE, M, K, P) == expect


def test_gemv_rejects_null_and_misaligned(lib):
    assert lib.seedmm_gemv(None, FAKE, FAKE, 0, FAKE, FAKE, 16, 16, 4) == -1
    assert lib.seedmm_gemv(FAKE, FAKE, FAKE, 0, None, FAKE, 16, 16, 4) == -1
    assert lib.seedmm_gemv(FAKE, FAKE, FAKE, 0, FAKE + 4, FAKE, 16, 16, 4) == -2


def test_gemv_ex_rejects(lib):
    f = lib.seedmm_gemv_ex
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 7, 16, FAKE, 16, 16, 16, 4, 1, None) == -1   # dtype
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 1, 8, FAKE, 16, 16, 16, 4, 1, None) == -1    # ldx < K
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 1, 16, FAKE, 8, 16, 16, 4, 1, None) == -1    # ldy < M
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 1, 20, FAKE, 16, 16, 16, 4, 2, None) == -2   # bf16 ldx % 8
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 0, 18, FAKE, 16, 16, 16, 4, 2, None) == -2   # f32 ldx % 4
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 1, 16, FAKE, 16, 16, 16, 4, -1, None) == -1  # N < 0
    # empty problems are a no-op success
    assert f(None, None, None, 0, None, 1, 16, None, 16, 0, 16, 4, 4, None) == 0
    assert f(None, None, None, 0, None, 1, 16, None, 16, 16, 16, 4, 0, None) == 0


def test_reconstruct_rejects(lib):
    f = lib.seedmm_reconstruct
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 3, 16, 16, 4, None) == -1     # dtype
    assert f(FAKE, FAKE, FAKE, 0, FAKE, 0, 16, 15, 4, None) == -1     # K
    assert f(FAKE, FAKE, FAKE, 0, FAKE + 2, 0, 16, 16, 4, None) == -2  # W alignment
    assert f(None, None, None, 0, None, 0, 0, 16, 4, None) == 0       # empty


def _mat():
    from pseudo_random_weight_amd.seedmm import SeedMat
    return SeedMat(FAKE, FAKE, FAKE, FAKE)


def test_moe_rejects_and_workspace(lib):
    f = lib.seedmm_moe
    ws = lib.seedmm_moe_workspace_bytes(64, 8, 100, 2048, 1024)
    assert ws > 64 * 8 * (1024 * 2 + 2048 * 4)
    assert lib.seedmm_moe_workspace_bytes(128, 8, 100, 2048, 1024) > ws
    assert lib.seedmm_moe_workspace_bytes(-1, 8, 100, 2048, 1024) == 0
    m = _mat()
    args = lambda T=4, k=2, E=8, H=64, I=32, P=4, wsb=ws, x=FAKE: (
        FAKE, FAKE, T, k, x, FAKE, E, H, I, P, m, m, m, FAKE, wsb, None)
    assert f(*args(k=9)) == -1               # top_k > E
    assert f(*args(k=0)) == -1
    assert f(*args(H=60)) == -1              # H % 8
    assert f(*args(P=5)) == -1
    assert f(*args(E=0)) == -1
    assert f(*args(wsb=16)) == -3            # workspace too small
    assert f(*args(x=FAKE + 2)) == -2        # x misaligned
    assert f(*args(T=0)) == 0                # empty batch: no-op
    # pair indices t * top_k + slot are int32: 2^31 pairs or more are refused
    assert lib.seedmm_moe_workspace_bytes(1 << 25, 64, 100, 8, 8) == 0
    assert lib.seedmm_moe_workspace_bytes((1 << 25) - 1, 64, 100, 8, 8) > 0
    assert f(*args(T=1 << 25, k=64, E=100, H=8, I=8, wsb=1 << 62)) == -1


def test_dispatch_rejects(lib):
    assert lib.seedmm_moe_dispatch(FAKE, 4, 0, 8, FAKE, FAKE, None) == -1
    assert lib.seedmm_moe_dispatch(FAKE, -1, 2, 8, FAKE, FAKE, None) == -1
    assert lib.seedmm_moe_dispatch(FAKE, 4, 2, 0, FAKE, FAKE, None) == -1
    assert lib.seedmm_moe_dispatch(FAKE, 1 << 25, 64, 8, FAKE, FAKE, None) == -1


def test_binding_has_no_fallback():
    src = open(os.path.join(ROOT, "pseudo_random_weight_amd", "seedmm.py")).read()
    assert "import oracle" not in src and "from oracle" not in src
    assert "raise ImportError" in src


def test_search_rejects(lib):
    f = lib.seedmm_search
    # (W, ldw, colw, M, K, P, exp_bias, seeds, coefs, codes, err, table, stream)
    T = FAKE   # a 256-byte aligned table address, never dereferenced
    assert f(FAKE, 12, None, 4, 12, 4, -4, FAKE, FAKE, FAKE, None, T, None) == -1    # K % 8
    assert f(FAKE, 16, None, 4, 16, 5, -4, FAKE, FAKE, FAKE, None, T, None) == -1    # P
    assert f(FAKE, 16, None, 4, 16, 4, 101, FAKE, FAKE, FAKE, None, T, None) == -1   # exp_bias
    assert f(FAKE, 8, None, 4, 16, 4, -4, FAKE, FAKE, FAKE, None, T, None) == -1     # ldw < K
    assert f(None, 16, None, 4, 16, 4, -4, FAKE, FAKE, FAKE, None, T, None) == -1    # null W
    assert f(FAKE, 16, None, 4, 16, 4, -4, FAKE, None, FAKE, None, T, None) == -1    # null coefs
    assert f(FAKE, 16, None, 4, 16, 4, -4, FAKE, FAKE, FAKE, None, None, None) == -1  # no table
    assert f(FAKE, 16, None, 4, 16, 4, -4, FAKE, FAKE, FAKE, None, T + 16, None) == -2  # table align
    assert f(None, 16, None, 0, 16, 4, -4, None, None, None, None, None, None) == 0  # empty


def test_search_table_size_and_prepare_rejects(lib):
    n4, n3 = lib.seedmm_search_table_bytes(4), lib.seedmm_search_table_bytes(3)
    assert n4 > n3 > 8_000_000 and n4 % 256 == 0 and n3 % 256 == 0
    assert lib.seedmm_search_table_bytes(5) == 0
    g = lib.seedmm_search_prepare
    assert g(5, FAKE, n4, None) == -1           # P
    assert g(4, None, n4, None) == -1           # null table
    assert g(4, FAKE, n4 - 1, None) == -1       # too small
    assert g(4, FAKE + 16, n4, None) == -2      # alignment


def test_moe_ex_rejects(lib):
    from pseudo_random_weight_amd.seedmm import SeedMat, SeedSide
    m = SeedMat(FAKE, FAKE, FAKE, FAKE)
    ws = lib.seedmm_moe_workspace_bytes(4, 2, 8, 64, 64)
    f = lib.seedmm_moe_ex

    def call(P=4, mask=None, side=None):
        return f(FAKE, FAKE, 4, 2, FAKE, FAKE, 8, 64, 64, P, mask, m, m, m, FAKE, ws, FAKE,
                 None if side is None else ctypes.byref(side))
    assert call(P=0) == -1                                   # mixed without a mask
    assert call(P=4, mask=FAKE) == -1                        # a mask with one P
    assert call(P=5) == -1
    assert call(side=SeedSide(FAKE + 256, None, FAKE)) == -1  # side stream without a fork
    assert call(side=SeedSide(FAKE, FAKE, FAKE)) == -1        # side stream = hip_stream


def test_moe_mixed_rejects_a_missing_mask(lib):
    from pseudo_random_weight_amd.seedmm import SeedMat
    m = SeedMat(FAKE, FAKE, FAKE, FAKE)
    assert lib.seedmm_moe_mixed(FAKE, FAKE, 4, 2, FAKE, FAKE, 8, 64, 64, None, m, m, m,
                                FAKE, 1 << 30, None) == -1


def test_binding_stream_sizes_match_the_generated_streams():
    """The binding's length check uses the stream sizes the layout fixes: they equal the
    lengths of generated stacks, uniform and mixed."""
    import numpy as np
    import synth
    from pseudo_random_weight_amd import seedmm
    for (E, M, K, P) in [(1, 256, 512, 4), (3, 24, 16, 3), (5, 64, 128, 4)]:
        m = synth.seed_matrix(synth.config_seed(0), f"sz{E}{P}", M, K, P, E)
        need = seedmm.stream_sizes(E, M, K, P)
        assert need == {k: m[k].size for k in ("seeds", "coefs", "codes")}
    Ps = [4, 3, 3, 4, 3]
    mm = synth.seed_matrix_mixed(synth.config_seed(0), "szmix", 32, 64, Ps)
    assert seedmm.stream_sizes(5, 32, 64, Ps) == {k: mm[k].size for k in ("seeds", "coefs", "codes")}


def test_binding_refuses_short_streams():
    """A P = 3 stack passed as P = 4 (its coefficient stream is a quarter short) is refused
    before any launch, as is a missing expert."""
    import numpy as np
    import torch
    import synth
    from pseudo_random_weight_amd import seedmm
    E, M, K = 4, 32, 64
    m3 = synth.seed_matrix(synth.config_seed(0), "short", M, K, 3, E)
    t = {k: torch.from_numpy(np.ascontiguousarray(m3[k]).view(np.uint8 if k == "codes" else np.int16))
         for k in ("seeds", "coefs", "codes")}
    t["exp_bias"] = torch.from_numpy(m3["exp_bias"])
    seedmm._check_streams(t, E, M, K, 3, "gate")                  # fits
    with pytest.raises(ValueError, match="coefs"):
        seedmm._check_streams(t, E, M, K, 4, "gate")
    with pytest.raises(ValueError, match="seeds"):
        seedmm._check_streams(t, E + 1, M, K, 3, "gate")
    seedmm._check_streams(t, E, M, K, 4, "gate", exact_coefs=False)   # mixed without Ps


def test_noalloc_refuses_before_running(lib):
    """seedmm_moe_noalloc checks the batch against its static scratch before it touches
    the device: a batch needing more than 8 MiB is refused (no GPU needed)."""
    from pseudo_random_weight_amd.seedmm import SeedMat, NOALLOC_SCRATCH_BYTES, ESCRATCH
    m = SeedMat(FAKE, FAKE, FAKE, FAKE)
    assert lib.seedmm_moe_workspace_bytes(128, 8, 100, 2048, 1024) > NOALLOC_SCRATCH_BYTES
    f = lib.seedmm_moe_noalloc
    assert f(FAKE, FAKE, 128, 8, FAKE, FAKE, 100, 2048, 1024, 4, m, m, m, None) == ESCRATCH
    assert f(FAKE, FAKE, 4, 2, FAKE, FAKE, 8, 64, 64, 5, m, m, m, None) == -1    # P
    assert f(FAKE, FAKE, 4, 0, FAKE, FAKE, 8, 64, 64, 4, m, m, m, None) == -1    # top_k
    assert lib.seedmm_strerror(ESCRATCH) != lib.seedmm_strerror(99)


def test_binding_checks_topk_ids_on_the_host():
    """check_topk_ids (and moe's check_ids=True) refuses ids outside [0, E) and an expert
    named twice by one token, naming the token; valid routings pass."""
    import torch
    from pseudo_random_weight_amd import seedmm
    ok = torch.tensor([[0, 3, 7], [7, 1, 2]], dtype=torch.int32)
    seedmm.check_topk_ids(ok, 8)
    seedmm.check_topk_ids(torch.tensor([[5]], dtype=torch.int32), 8)
    for bad, what in (([[0, 3, 8], [1, 2, 4]], "topk_ids[0]"), ([[0, 1, 2], [-1, 2, 3]], "topk_ids[1]"),
                      ([[0, 1, 2], [4, 5, 4]], "topk_ids[1]")):
        with pytest.raises(ValueError, match=re.escape(what)):
            seedmm.check_topk_ids(torch.tensor(bad, dtype=torch.int32), 8)
    with pytest.raises(ValueError):
        seedmm.check_topk_ids(torch.tensor([1, 2], dtype=torch.int32), 8)
