"""GPU check of seedmm_moe_noalloc, the layer call whose scratch is the library's static
device array: through the C ABI, its output equals seedmm_moe's (caller workspace) bit
for bit, on consecutive calls whose second input is smaller than the first (the array
keeps the first call's contents), and on a one-token call; a batch whose scratch would
exceed the array is refused before anything runs."""
import ctypes
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _dev(mat):
    import torch
    return {
        "seeds": torch.from_numpy(mat["seeds"].view(np.int16).copy()).view(torch.uint16).cuda(),
        "coefs": torch.from_numpy(mat["coefs"].view(np.int16).copy()).view(torch.uint16).cuda(),
        "codes": torch.from_numpy(mat["codes"].copy()).cuda(),
        "exp_bias": torch.from_numpy(mat["exp_bias"].copy()).cuda(),
    }


def _noalloc(sm, ids_t, w_t, xt, y, E, H, I, P, mats):
    import torch
    T, k = ids_t.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = sm.lib().seedmm_moe_noalloc(p(ids_t), p(w_t), T, k, p(xt), p(y), E, H, I, P,
                                     *[sm._seedmat(m) for m in mats],
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("E,H,I,P,k,Ts", [
    (100, 2048, 1024, 4, 8, (64, 5, 1)),   # the decode layer: 5.3 MB of scratch, then less
    (8, 256, 256, 3, 2, (600, 40)),        # prefill kernels, then decode kernels
])
def test_noalloc_matches_the_workspace_call(E, H, I, P, k, Ts):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from pseudo_random_weight_amd import seedmm as sm
    base = synth.config_seed(30)
    mats = [_dev(synth.seed_matrix(base, f"na{E}.{n}", *((I, H) if n != "down" else (H, I)), P, E))
            for n in ("gate", "up", "down")]
    for T in Ts:
        say("noalloc", E, H, I, P, k, T)
        ids, w = synth.route_topk(base, f"na.r{E}.{T}", T, E, k)
        x = synth.bf16_bits(synth.normal_f32(base, f"na.x{E}.{T}", (T, H)))
        ids_t, w_t = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
        xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        assert sm.moe_workspace_bytes(T, k, E, H, I) <= sm.NOALLOC_SCRATCH_BYTES
        st = _noalloc(sm, ids_t, w_t, xt, y, E, H, I, P, mats)
        assert st == sm.OK, sm.lib().seedmm_strerror(st)
        y_ref = sm.moe(ids_t, w_t, xt, E, H, I, P, *mats)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.cpu().numpy().view(np.uint32)), T


def test_noalloc_refuses_a_batch_beyond_its_scratch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from pseudo_random_weight_amd import seedmm as sm
    E, H, I, P, k = 100, 2048, 1024, 4, 8
    T = 128
    assert sm.moe_workspace_bytes(T, k, E, H, I) > sm.NOALLOC_SCRATCH_BYTES
    base = synth.config_seed(30)
    mats = [_dev(synth.seed_matrix(base, f"nb.{n}", *((I, H) if n != "down" else (H, I)), P, 2))
            for n in ("gate", "up", "down")]
    ids_t = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    w_t = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    xt = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
    assert _noalloc(sm, ids_t, w_t, xt, y, E, H, I, P, mats) == sm.ESCRATCH
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())            # nothing ran
