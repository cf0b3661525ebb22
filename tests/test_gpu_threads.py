"""GPU check that the library keeps no state between calls: host threads that call the
layer at the same time, each with its own stream, workspace, output and (for half of
them) its own second stream and events, get the same bits as one thread calling alone.
The batches cover the one-token, decode and prefill kernels."""
import sys
import threading

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


def test_concurrent_host_threads_match_one_thread():
    import torch
    from pseudo_random_weight_amd import seedmm as sm
    E, H, I, P, k = 8, 256, 256, 4, 2
    base = synth.config_seed(51)
    mats = [_dev(synth.seed_matrix(base, f"thr.{n}", *((I, H) if n != "down" else (H, I)), P, E,
                                   exp_bias=eb))
            for n, eb in (("gate", -20), ("up", -19), ("down", -18))]
    cases = []
    for c, T in enumerate((1, 5, 64, 300)):   # one token, decode, decode, prefill
        ids, w = synth.route_topk(base, f"thr.r{c}", T, E, k)
        x = synth.bf16_bits(synth.normal_f32(base, f"thr.x{c}", (T, H)))
        cases.append((torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(),
                      torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()))
    say("threads: single-thread references")
    ref = [sm.moe(i, w, x, E, H, I, P, *mats).cpu() for (i, w, x) in cases]
    torch.cuda.synchronize()

    errors, done = [], []

    def worker(tid):
        try:
            st = torch.cuda.Stream()
            side = sm.SideStream() if tid % 2 else None
            with torch.cuda.stream(st):
                bufs = [(torch.empty((c[2].shape[0], H), dtype=torch.float32, device="cuda"),
                         torch.empty(sm.moe_workspace_bytes(c[2].shape[0], k, E, H, I),
                                     dtype=torch.uint8, device="cuda")) for c in cases]
            for it in range(16):
                c = (it + tid) % len(cases)
                ids, w, x = cases[c]
                y, ws = bufs[c]
                sm.moe(ids, w, x, E, H, I, P, *mats, y=y, workspace=ws, stream=st, side=side)
                st.synchronize()
                if not torch.equal(y.cpu().view(torch.int32), ref[c].view(torch.int32)):
                    errors.append((tid, it, c))
            done.append(tid)
        except Exception as exc:   # reported by the main thread
            errors.append((tid, repr(exc)))

    say("threads: 4 concurrent callers x 16 calls")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=90)
    assert sorted(done) == [0, 1, 2, 3], (done, errors)
    assert not errors, errors
