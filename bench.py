#!/usr/bin/env python
"""Benchmark of the seed-decoding MoE layer on one MI355X.

A step is one decode pass of a routed mixture-of-experts layer whose expert weights
are SeedLM seeds: 100 SwiGLU experts 2048 -> 1024 -> 2048, P = 4, top-8 softmax
routing, T bf16 tokens (default 64): dispatch, fused gate/up + SwiGLU, down, ordered
combine.  Inputs are synthetic (seeded generator), resident in HBM before timing;
the weights rotate over replicas so every step reads its compressed weights from HBM,
not from the 256 MB Infinity Cache.

Two timed regions: eager launches with HIP events between the kernels (fresh routing
and activations every step) give the per-stage times and the roofline of the dominant
kernel (fused gate/up); HIP-graph replays of the whole layer call (six captured input
sets, each with its own routing and activations) give the step time, as a serving loop
that captures its decode step would run it (--eager times the eager launches instead).

Prints one JSON line: effective weights/s (distinct expert weights applied per second),
compressed HBM GB/s and its fraction of 8 TB/s, decode tokens/s, the roofline, and the
CPU oracle timed on a bounded sample of the same step; "encoder" adds the exhaustive
seed search's blocks/s on a 512 x 2048 matrix beside the oracle's search.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective weights/s + compressed HBM GB/s (% roofline); MoE-layer decode tok/s"
HBM_PEAK = 8.0e12                 # bytes/s, MI355X HBM3E
VALU_PEAK = 256 * 4 * 16 * 2.4e9  # lane-ops/s: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz


def ALG_OPS(P):
    """Algorithmic vector lane-ops per regenerated weight: P register states, P integer
    multiply-adds c * (s - 32768), and one power-of-two scale per block of 8 weights."""
    return 2 * P + 1.0 / 8
MFMA_PEAK = 2.5e15                 # flop/s, dense bf16 matrix cores
E, H, I, TOPK = 100, 2048, 1024, 8


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=64, help="decode batch T")
    ap.add_argument("--P", type=int, default=4, choices=(3, 4))
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-sweep", action="store_true", help="skip the T = 1, 4, 16 lines")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one plain device copy of this size (counter calibration)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of HIP-graph replays of the step")
    ap.add_argument("--no-encoder", action="store_true",
                    help="skip the seed-search (encoder) measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (single GEMV, one expert, P = 3, prefill)")
    ap.add_argument("--no-cache", action="store_true",
                    help="skip the host-resident experts with a device expert cache")
    ap.add_argument("--no-mixed", action="store_true",
                    help="skip the mixed P3/P4 layer measurement")
    return ap.parse_args()


def host_cpu():
    """CPU model and the cores this process may use (for the oracle baseline): the model
    name, vendor, family / model / stepping and core counts from /proc/cpuinfo."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if ":" not in line:
                    if info:
                        break
                    continue
                k, v = (p.strip() for p in line.split(":", 1))
                if k in ("model name", "vendor_id", "cpu family", "model", "stepping",
                         "cpu MHz", "cache size", "cpu cores", "siblings") and k not in info:
                    info[k] = v
    except OSError:
        pass
    return {"model": info.get("model name"), "cpuinfo": info,
            "nproc": len(os.sched_getaffinity(0)), "logical_cpus": os.cpu_count()}


def compressed_bytes_per_matrix(P):
    nblk = H * I // 8
    return nblk * 2 + (nblk * P + 3) // 4 * 2 + (nblk + 1) // 2


def read_traffic(kernel_tag):
    """HBM bytes per launch from the committed counter summary, if it still matches the
    kernel sources (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in ("seedmm.hip", "seed_decode.hpp"):
        with open(os.path.join(ROOT, "pseudo_random_weight_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()[:16]
    vals = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != digest:
        return None
    key = f"{kernel_tag}.bytes_per_launch"
    return float(vals[key]) if key in vals else None


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime (the library records them between its
    kernels; torch's Event wrapper cannot time events it did not record itself)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.live = []

    def create(self):
        h = self.ct.c_void_p()
        rc = self.hip.hipEventCreate(self.ct.byref(h))
        assert rc == 0, f"hipEventCreate failed ({rc})"
        self.live.append(h.value)
        return h.value

    def ms(self, a, b):
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), self.ct.c_void_p(a), self.ct.c_void_p(b))
        assert rc == 0, f"hipEventElapsedTime failed ({rc})"
        return out.value

    def close(self):
        for h in self.live:
            self.hip.hipEventDestroy(self.ct.c_void_p(h))
        self.live = []


def warm_replays(torch, graphs, seconds=0.03):
    """Untimed replays until about `seconds` of steps have run.  The clocks drop while the
    GPU idles (graph capture, synchronisations) and need ~10 ms of load to come back; a
    timed pass started cold measured ~10% slower steps."""
    t_w = time.perf_counter()
    for s_ in range(4):
        graphs[s_ % len(graphs)].replay()
    torch.cuda.synchronize()
    est = max((time.perf_counter() - t_w) / 4, 1e-6)
    for s_ in range(int(seconds / est)):
        graphs[s_ % len(graphs)].replay()
    torch.cuda.synchronize()


def graph_step(torch, calls, steps):
    """Wall time per step of HIP-graph replays of `calls` (one captured graph per input
    set, cycled), after an untimed warm-up."""
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    graphs = []
    for c in calls:
        G = torch.cuda.CUDAGraph()
        with torch.cuda.graph(G):
            c()
        graphs.append(G)
    warm_replays(torch, graphs)
    t0 = time.perf_counter()
    for s_ in range(steps):
        graphs[s_ % len(graphs)].replay()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    del graphs
    return t


def config_lines(torch, seedmm, synth, reps, to_dev, P, side):
    """One timed figure for each of the other workloads: the single matrix-vector product
    (256 x 512, fp32 x), one SwiGLU expert (2048 -> 768 -> 2048) at 1 and 8 tokens, the
    P = 3 layer at 1 and 16 tokens, and 4096-token prefill through the bench's own layer
    (`reps`, whose streams have P coefficients per block).  Multi-token layer calls run
    half their expert launches on the caller's second stream `side`."""
    dev = torch.device("cuda:0")
    out = {}
    # C1: back-to-back launches on the default stream (launch overhead included), on one
    # matrix (warm caches) and rotating over 8192 copies (604 MB, beyond the 256 MB cache)
    M1, K1, R1 = 256, 512, 8192
    base = synth.config_seed(0)
    m = synth.seed_matrix(base, "bench.C1", M1, K1, 4)
    seeds = torch.from_numpy(np.tile(m["seeds"].view(np.int16), R1).reshape(R1, -1)).view(torch.uint16).to(dev)
    coefs = torch.from_numpy(np.tile(m["coefs"].view(np.int16), R1).reshape(R1, -1)).view(torch.uint16).to(dev)
    codes = torch.from_numpy(np.tile(m["codes"], R1).reshape(R1, -1)).to(dev)
    mats = [{"seeds": seeds[r], "coefs": coefs[r], "codes": codes[r], "exp_bias_host": m["exp_bias"]}
            for r in range(R1)]
    x = torch.from_numpy(synth.normal_f32(base, "bench.C1.x", (K1,))).to(dev)
    y = torch.empty(M1, dtype=torch.float32, device=dev)

    def launches(n, rot):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            seedmm.gemv(mats[i % R1 if rot else 0], x, M1, K1, 4, y=y)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    launches(500, False)
    hot = launches(2000, False)
    launches(R1, True)
    cold = launches(R1, True)
    out["C1_gemv_256x512_fp32"] = {"us_per_launch_hot": hot * 1e6, "us_per_launch_cold": cold * 1e6,
                                   "weights_per_s_cold": M1 * K1 / cold, "cold_copies": R1}
    del seeds, coefs, codes, mats
    # C2: one expert, top-1 with weight 1 (graph replays)
    b2 = synth.config_seed(1)
    ex = {n: to_dev(synth.seed_matrix(b2, f"bench.C2.{n}", *((768, 2048) if n != "down" else (2048, 768)), 4, 1))
          for n in ("gate", "up", "down")}
    c2 = {}
    for T2 in (1, 8):
        ids = torch.zeros((T2, 1), dtype=torch.int32, device=dev)
        w = torch.ones((T2, 1), dtype=torch.float32, device=dev)
        xs = [torch.from_numpy(synth.bf16_bits(synth.normal_f32(b2, f"bench.C2.x{T2}.{g}", (T2, 2048))).view(np.int16)
                               ).view(torch.bfloat16).to(dev) for g in range(4)]
        y2 = torch.empty((T2, 2048), dtype=torch.float32, device=dev)
        ws = torch.empty(seedmm.moe_workspace_bytes(T2, 1, 1, 2048, 768), dtype=torch.uint8, device=dev)
        calls = [lambda xg=xg: seedmm.moe(ids, w, xg, 1, 2048, 768, 4, ex["gate"], ex["up"], ex["down"],
                                          y=y2, workspace=ws) for xg in xs]
        t = graph_step(torch, calls, 200)
        c2[f"T{T2}_us"] = t * 1e6
        c2[f"T{T2}_weights_per_s"] = 3 * 2048 * 768 / t
    out["C2_expert_2048x768_P4"] = c2
    del ex
    # C4: the 100-expert layer with P = 3
    b4 = synth.config_seed(3)
    l3 = [{n: to_dev(synth.seed_matrix(b4, n, *((I, H) if n != "down" else (H, I)), 3, E))
           for n in ("gate", "up", "down")}]
    for _ in range(2):
        l3.append({n: {k: v.clone() for k, v in mm.items()} for n, mm in l3[0].items()})
    c4 = {}
    for T4 in (1, 16):
        calls, dist = [], []
        y4 = torch.empty((T4, H), dtype=torch.float32, device=dev)
        ws = torch.empty(seedmm.moe_workspace_bytes(T4, TOPK, E, H, I), dtype=torch.uint8, device=dev)
        for g in range(6):
            ids, w = synth.route_topk(b4, f"bench.C4.r{T4}.{g}", T4, E, TOPK)
            dist.append(len(np.unique(ids)))
            xg = torch.from_numpy(synth.bf16_bits(synth.normal_f32(b4, f"bench.C4.x{T4}.{g}", (T4, H))).view(np.int16)
                                  ).view(torch.bfloat16).to(dev)
            r = l3[g % 3]
            calls.append(lambda i=torch.from_numpy(ids).to(dev), wt=torch.from_numpy(w).to(dev), xg=xg, r=r:
                         seedmm.moe(i, wt, xg, E, H, I, 3, r["gate"], r["up"], r["down"], y=y4, workspace=ws,
                                    side=side))
        t = graph_step(torch, calls, 100 if T4 == 1 else 50)
        c4[f"T{T4}_us"] = t * 1e6
        c4[f"T{T4}_weights_per_s"] = np.mean(dist) * 3 * H * I / t
        c4[f"T{T4}_tok_s"] = T4 / t
    out["C4_moe_layer_P3"] = c4
    del l3
    # C5: 4096-token prefill through the headline's layer (its weight copies, its P)
    T5 = 4096
    y5 = torch.empty((T5, H), dtype=torch.float32, device=dev)
    ws = torch.empty(seedmm.moe_workspace_bytes(T5, TOPK, E, H, I), dtype=torch.uint8, device=dev)
    b5 = synth.config_seed(2)
    calls = []
    for g in range(3):
        ids, w = synth.route_topk(b5, f"bench.C5.r{g}", T5, E, TOPK)
        xg = torch.from_numpy(synth.bf16_bits(synth.normal_f32(b5, f"bench.C5.x{g}", (T5, H))).view(np.int16)
                              ).view(torch.bfloat16).to(dev)
        r = reps[g % len(reps)]
        calls.append(lambda i=torch.from_numpy(ids).to(dev), wt=torch.from_numpy(w).to(dev), xg=xg, r=r:
                     seedmm.moe(i, wt, xg, E, H, I, P, r["gate"], r["up"], r["down"], y=y5, workspace=ws,
                                side=side))
    t = graph_step(torch, calls, 10)
    flops = 2.0 * T5 * TOPK * 3 * H * I
    out[f"C5_prefill_T4096_P{P}"] = {"ms_per_step": t * 1e3, "tok_s": T5 / t,
                                  "weights_per_s": E * 3 * H * I / t,
                                  "mfma_tflops": flops / t / 1e12, "mfma_frac": flops / t / MFMA_PEAK}
    return out


def mixed_bench(torch, seedmm, synth, dev, T, replicas, to_dev, side, steps=30):
    """The same layer as a mixed pack: a seeded random half of the experts P = 4, the
    rest P = 3 (seedmm_moe_mixed); HIP-graph replays over six input sets and the weight
    replicas, as for the headline step."""
    base = synth.config_seed(11)
    Ps = [4 if v else 3 for v in (synth.uniform_u64(base, "mix.P", E) & np.uint64(1))]
    host = {n: synth.seed_matrix_mixed(base, f"mix.{n}", *((I, H) if n != "down" else (H, I)), Ps)
            for n in ("gate", "up", "down")}
    reps = [{n: to_dev(m) for n, m in host.items()}]
    for _ in range(replicas - 1):
        reps.append({n: {k: v.clone() for k, v in m.items()} for n, m in reps[0].items()})
    mask = seedmm.p4_mask(Ps, dev)
    ids_l, w_l, x_l, dist = [], [], [], []
    for g in range(6):
        i, w = synth.route_topk(base, f"mix.r{g}", T, E, TOPK)
        x = synth.bf16_bits(synth.normal_f32(base, f"mix.x{g}", (T, H)))
        ids_l.append(torch.from_numpy(i).to(dev)), w_l.append(torch.from_numpy(w).to(dev))
        x_l.append(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev))
        dist.append(np.unique(i))
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(seedmm.moe_workspace_bytes(T, TOPK, E, H, I), dtype=torch.uint8, device=dev)

    def call(g):
        r = reps[g % len(reps)]
        seedmm.moe_mixed(ids_l[g], w_l[g], x_l[g], E, H, I, mask, r["gate"], r["up"], r["down"],
                         y=y, workspace=ws, Ps=Ps, side=side)

    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        for g in range(6):
            call(g)
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    graphs = []
    for g in range(6):
        G = torch.cuda.CUDAGraph()
        with torch.cuda.graph(G):
            call(g)
        graphs.append(G)
    for s_ in range(6):
        graphs[s_].replay()
    torch.cuda.synchronize()
    warm_replays(torch, graphs)
    t0 = time.perf_counter()
    for s_ in range(steps):
        graphs[s_ % 6].replay()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    nblk = H * I // 8
    wts = np.mean([len(d) for d in dist]) * 3 * H * I
    cb = np.mean([sum(3 * (nblk * 2 + nblk * Ps[e] // 4 * 2 + nblk // 2) for e in d) for d in dist])
    return {"workload": f"moe_layer_decode, mixed pack ({sum(p == 4 for p in Ps)} P4 / "
                        f"{sum(p == 3 for p in Ps)} P3 experts), T={T}",
            "bits_per_weight": float(np.mean([16 + 4 * p + 4 for p in Ps]) / 8),
            "ms_per_step": t * 1e3, "weights_per_s": wts / t, "compressed_GBps": cb / t / 1e9,
            "tok_s": T / t}


def cache_bench(torch, seedmm, synth, host, P, steps=200, warmup=30, S=33):
    """Experts in pinned host memory behind an S-slot device cache (seedmm_cache_moe),
    one-token decode, eager calls (the cache plans each call on the host).  Two routing
    recipes: i.i.d. router logits, and a hot third of the experts taking ~85% of the
    router choices.  Also the host-to-device rate of one large pinned copy."""
    dev = torch.device("cuda:0")
    base = synth.config_seed(13)
    cache = seedmm.ExpertCache(host, E, H, I, P, S)
    y = torch.empty((1, H), dtype=torch.float32, device=dev)
    ws = torch.empty(seedmm.moe_workspace_bytes(1, TOPK, E, H, I), dtype=torch.uint8, device=dev)
    out = {"workload": f"moe_layer_decode T=1, experts in pinned host memory, {S} of {E} "
                       f"experts cached on the device (LRU)",
           "slots": S, "slot_MB": 3 * compressed_bytes_per_matrix(P) / 1e6}
    hb, _ = synth.hot_bias(base, E)
    for name, bias in (("uniform", None), ("hot_third", hb)):
        n = warmup + steps
        ids, w = synth.route_topk(base, f"cache.{name}", n, E, TOPK, bias=bias)
        x = synth.bf16_bits(synth.normal_f32(base, f"cache.x.{name}", (n, H)))
        ids_d = torch.from_numpy(ids).to(dev)
        w_d = torch.from_numpy(w).to(dev)
        x_d = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        cache.reset()

        def call(s):
            cache.moe(ids[s:s + 1], ids_d[s:s + 1], w_d[s:s + 1], x_d[s:s + 1], y=y,
                      workspace=ws)

        for s in range(warmup):
            call(s)
        torch.cuda.synchronize()
        st0 = cache.stats()
        t0 = time.perf_counter()
        for s in range(warmup, n):
            call(s)
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / steps
        st1 = cache.stats()
        d = {k: st1[k] - st0[k] for k in st1}
        out[name] = {"ms_per_step": t * 1e3, "tok_s": 1.0 / t,
                     "hit_rate": d["hits"] / max(d["uses"], 1),
                     "loads_per_step": d["misses"] / steps,
                     "h2d_GBps": d["bytes"] / steps / t / 1e9}
    # the same one-token calls with every expert resident (eager, for comparison)
    devm = {}
    for nme, m in host.items():
        devm[nme] = {"seeds": torch.from_numpy(m["seeds"].view(np.int16)).view(torch.uint16).to(dev),
                     "coefs": torch.from_numpy(m["coefs"].view(np.int16)).view(torch.uint16).to(dev),
                     "codes": torch.from_numpy(m["codes"]).to(dev),
                     "exp_bias": torch.from_numpy(m["exp_bias"]).to(dev)}
    for s in range(warmup):
        seedmm.moe(ids_d[s:s + 1], w_d[s:s + 1], x_d[s:s + 1], E, H, I, P, devm["gate"],
                   devm["up"], devm["down"], y=y, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(warmup, warmup + steps):
        seedmm.moe(ids_d[s:s + 1], w_d[s:s + 1], x_d[s:s + 1], E, H, I, P, devm["gate"],
                   devm["up"], devm["down"], y=y, workspace=ws)
    torch.cuda.synchronize()
    out["resident_eager_ms_per_step"] = (time.perf_counter() - t0) / steps * 1e3
    # host-to-device rate of one 256 MiB pinned copy
    src = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    out["pinned_h2d_GBps"] = 3 * (256 << 20) / (time.perf_counter() - t0) / 1e9
    del cache, devm, src, dst
    return out


def encoder_bench(torch, seedmm, synth, P, no_cpu):
    """The exhaustive seed search (seedmm_search) on a synthetic fp32 matrix of 512 rows x
    2048 columns (weights ~N(0, 0.02^2), exp_bias -4): blocks encoded per second, with
    the oracle's search timed on a 64-block sample of the same matrix."""
    M, K, eb = 512, 2048, -4
    W = (synth.normal_f32(synth.config_seed(7), "encoder.W", (M, K)) * 0.02).astype(np.float32)
    Wd = torch.from_numpy(W).cuda()
    seedmm.search(Wd[:4], P, eb)                      # warm-up (module load, first launch)
    torch.cuda.synchronize()
    reps, t = 3, 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        enc = seedmm.search(Wd, P, eb)
        torch.cuda.synchronize()
        t += time.perf_counter() - t0
    t /= reps
    nblk = M * K // 8
    res = {"workload": f"exhaustive seed search, fp32 W {M}x{K}, P={P}, exp_bias {eb}",
           "blocks": nblk, "s_per_matrix": t, "blocks_per_s": nblk / t,
           "seed_trials_per_s": nblk * 65535 / t,
           "mean_block_sq_err": float(enc["err"].mean())}
    if not no_cpu:
        import oracle
        t0 = time.perf_counter()
        oracle.search_matrix(W[:1, :512], P, eb)      # 64 blocks
        tc = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": 64 / tc, "unit": "blocks/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": "oracle search of the first 64 blocks of the matrix"}
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from pseudo_random_weight_amd import seedmm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    P, T = args.P, args.tokens
    base = synth.config_seed(2 if P == 4 else 3)

    def to_dev(m):
        return {"seeds": torch.from_numpy(m["seeds"].view(np.int16)).view(torch.uint16).to(dev),
                "coefs": torch.from_numpy(m["coefs"].view(np.int16)).view(torch.uint16).to(dev),
                "codes": torch.from_numpy(m["codes"]).to(dev),
                "exp_bias": torch.from_numpy(m["exp_bias"]).to(dev)}

    hipev = HipEvents()
    # the caller-owned second stream and fork / join events of the layer calls
    side = seedmm.SideStream(dev)
    host = {n: synth.seed_matrix(base, n, *( (I, H) if n != "down" else (H, I) ), P, E)
            for n in ("gate", "up", "down")}
    reps = []
    first = {n: to_dev(m) for n, m in host.items()}
    reps.append(first)
    for _ in range(args.replicas - 1):
        reps.append({n: {k: v.clone() for k, v in m.items()} for n, m in first.items()})
    layer_bytes = 3 * E * compressed_bytes_per_matrix(P)

    nsteps_total = args.warmup + args.steps

    def make_batches(T, n):
        ids, ws, xs = [], [], []
        for s in range(n):
            i, w = synth.route_topk(base, f"router.T{T}.s{s}", T, E, TOPK)
            x = synth.bf16_bits(synth.normal_f32(base, f"x.T{T}.s{s}", (T, H)))
            ids.append(i), ws.append(w), xs.append(x)
        return (torch.from_numpy(np.stack(ids)).to(dev), torch.from_numpy(np.stack(ws)).to(dev),
                torch.from_numpy(np.stack(xs).view(np.int16)).view(torch.bfloat16).to(dev),
                ids)

    if args.calib_copy_mb:
        src = torch.empty(args.calib_copy_mb << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def run(T, warmup, steps, timed_events=True):
        ids_d, w_d, x_d, ids_h = make_batches(T, warmup + steps)
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws = torch.empty(seedmm.moe_workspace_bytes(T, TOPK, E, H, I), dtype=torch.uint8,
                         device=dev)
        evs = [[hipev.create() for _ in range(5)] for _ in range(steps)]

        def step(s, ev=None):
            r = reps[s % len(reps)]
            seedmm.moe(ids_d[s], w_d[s], x_d[s], E, H, I, P, r["gate"], r["up"], r["down"],
                       y=y, workspace=ws, events=ev)

        for s in range(warmup):
            step(s)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            step(warmup + s, evs[s] if timed_events else None)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        stages = np.zeros(4)
        if timed_events:
            for s in range(steps):
                for j in range(4):
                    stages[j] += hipev.ms(evs[s][j], evs[s][j + 1]) * 1e-3
            stages /= steps
        distinct = [len(np.unique(ids_h[warmup + s])) for s in range(steps)]
        return wall / steps, stages, np.array(distinct, dtype=np.float64), ids_h, x_d, w_d

    NB = 6   # input sets cycled by the graph replays (each paired with replica g % replicas)

    def run_graph(T, warmup, steps, nrep=None):
        """Per-step time of HIP-graph replays: one graph per input set captures the whole
        layer call (dispatch, gate/up, down, combine), as a serving loop would.  Returns
        the wall time per step (the timed region is bracketed by synchronizations), the
        distinct experts of each step and the 10th / 50th / 90th percentile of the
        per-replay times from events recorded between replays in a second, untimed pass
        (the events add a few microseconds per step).  nrep limits the weight
        replicas cycled (1: the same weights every step, a hot-cache figure)."""
        nrep = nrep or len(reps)
        ids_d, w_d, x_d, ids_h = make_batches(T, NB)
        y = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws = torch.empty(seedmm.moe_workspace_bytes(T, TOPK, E, H, I), dtype=torch.uint8,
                         device=dev)

        def call(g):
            r = reps[g % nrep]
            seedmm.moe(ids_d[g], w_d[g], x_d[g], E, H, I, P, r["gate"], r["up"], r["down"],
                       y=y, workspace=ws, side=side)

        warm = torch.cuda.Stream()
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            for g in range(NB):
                call(g)
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        graphs = []
        for g in range(NB):
            G = torch.cuda.CUDAGraph()
            with torch.cuda.graph(G):
                call(g)
            graphs.append(G)
        for s_ in range(warmup):
            graphs[s_ % NB].replay()
        torch.cuda.synchronize()
        warm_replays(torch, graphs)
        t0 = time.perf_counter()
        for s_ in range(steps):
            graphs[s_ % NB].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # per-replay spread from a second pass with an event between replays (events add
        # a few microseconds per step, so they stay out of the timed region above)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for s_ in range(steps):
            evs[s_].record()
            graphs[s_ % NB].replay()
        evs[steps].record()
        torch.cuda.synchronize()
        per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
        distinct = np.array([len(np.unique(ids_h[s_ % NB])) for s_ in range(steps)], dtype=np.float64)
        # the output of input set 0 (replica 0) from one more replay, for the oracle check
        graphs[0].replay()
        torch.cuda.synchronize()
        y0 = y.cpu().numpy()
        del graphs
        return wall / steps, distinct, np.percentile(per, [10, 50, 90]), y0

    # stage times and the roofline come from eager launches with HIP events around each
    # kernel; the step time is HIP-graph replays unless --eager.  The eager run gets 30
    # more warm-up steps: the first ~12 launches after start run ~10% slower (clock ramp)
    t_eager, stages, distinct, ids_h, x_d, w_d = run(T, args.warmup + 30, args.steps)
    pct = None
    if args.eager:
        t_step = t_eager
    else:
        t_step, distinct, pct, y_graph0 = run_graph(T, args.warmup, args.steps)
    w_per_mat = H * I
    weights = distinct.mean() * 3 * w_per_mat
    cbytes = distinct.mean() * 3 * compressed_bytes_per_matrix(P)
    value = weights / t_step
    gbps = cbytes / t_step

    # dominant kernel: fused gate/up (two thirds of the weights)
    t_gu = stages[1]
    gu_weights = distinct.mean() * 2 * w_per_mat
    alg_ops = gu_weights * ALG_OPS(P)
    traffic = read_traffic("gateup_T%d_P%d" % (T, P))
    traffic_note = ("calibrated FETCH_SIZE + WRITE_SIZE per launch read from "
                    "profiles/hbm_traffic.txt (rocprofv3 counter runs of the same kernel "
                    "sources, not this run)" if traffic is not None else
                    "no counter summary for the current kernel sources")
    prefill = T * TOPK >= 64 * E          # the library's switch to the LDS-tiled kernel
    if prefill:
        # the tiled kernel's products run on the matrix cores: useful bf16 flops
        flops = 2.0 * T * TOPK * 2 * H * I
        roofline = {"bound": "mfma", "achieved": flops / t_gu / 1e12, "peak": MFMA_PEAK / 1e12,
                    "unit": "TFLOP/s", "frac": flops / t_gu / MFMA_PEAK, "traffic": traffic,
                    "traffic_source": traffic_note,
                    "kernel": "k_wide<GATEUP> (prefill: fused gate/up + SwiGLU)",
                    "kernel_us": t_gu * 1e6}
    else:
        roofline = {"bound": "alu", "achieved": alg_ops / t_gu, "peak": VALU_PEAK,
                    "unit": "lane-op/s", "frac": alg_ops / t_gu / VALU_PEAK,
                    "traffic": traffic, "traffic_source": traffic_note,
                    "kernel": "k_mfma<GATEUP> (fused gate/up + SwiGLU)",
                    "alg_ops_per_weight": ALG_OPS(P),
                    "kernel_us": t_gu * 1e6,
                    "compressed_bytes_per_launch": distinct.mean() * 2 * compressed_bytes_per_matrix(P),
                    "hbm_frac_compressed": distinct.mean() * 2 * compressed_bytes_per_matrix(P)
                    / t_gu / HBM_PEAK}

    out = {
        "metric": METRIC, "value": value, "unit": "weights/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": t_step * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "moe_layer_prefill" if prefill else "moe_layer_decode", "experts": E, "top_k": TOPK, "hidden": H,
                   "intermediate": I, "P": P, "tokens": T, "activations": "bf16",
                   "weight_replicas": args.replicas, "layer_compressed_MB": layer_bytes / 1e6},
        "compressed_GBps": gbps / 1e9, "hbm_frac": gbps / HBM_PEAK, "tok_s": T / t_step,
        "distinct_experts_per_step": distinct.mean(),
        "stage_us": {"dispatch": stages[0] * 1e6, "gate_up": stages[1] * 1e6,
                     "down": stages[2] * 1e6, "combine": stages[3] * 1e6},
        "step_timing": "eager launches" if args.eager else
                       f"HIP-graph replays of the layer call ({NB} captured input sets)",
        "ms_per_step_eager": t_eager * 1e3,
        "roofline": roofline,
    }
    if pct is not None:
        out["step_ms_p10_p50_p90"] = [float(v) for v in pct]
        # the same graphs over a single weight copy: part of the layer stays in the
        # 256 MB last-level cache between steps (labelled, not the headline)
        t_hot, dis_hot, pct_hot, _ = run_graph(T, args.warmup, args.steps, nrep=1)
        out["hot_cache"] = {"ms_per_step": t_hot * 1e3,
                            "weights_per_s": dis_hot.mean() * 3 * w_per_mat / t_hot,
                            "step_ms_p10_p50_p90": [float(v) for v in pct_hot],
                            "note": "one weight copy reused every step"}

    if not args.no_sweep:
        sweep = {}
        for Ts in (1, 4, 16, 64):
            if Ts == T:
                continue
            ts, st, dis, *_ = run(Ts, 3, 20)
            if not args.eager:
                ts, dis, _, _ = run_graph(Ts, 3, 50)
            sweep[str(Ts)] = {"ms_per_step": ts * 1e3, "tok_s": Ts / ts,
                              "weights_per_s": dis.mean() * 3 * w_per_mat / ts,
                              "compressed_GBps": dis.mean() * 3 * compressed_bytes_per_matrix(P) / ts / 1e9,
                              "gate_up_us": st[1] * 1e6, "down_us": st[2] * 1e6,
                              # event timing: includes a few microseconds of event records
                              "gate_up_valu_frac": dis.mean() * 2 * w_per_mat * ALG_OPS(P)
                              / st[1] / VALU_PEAK}
        out["by_batch"] = sweep
        if "1" in sweep:
            # the one-token step: the vector-ALU fraction of its gate/up kernel (event
            # timing), next to the headline kernel's
            out["batch1_gate_up_valu_frac"] = sweep["1"]["gate_up_valu_frac"]

    if not args.no_configs:
        out["configs"] = config_lines(torch, seedmm, synth, reps, to_dev, P, side)

    if not args.no_mixed:
        out["mixed"] = mixed_bench(torch, seedmm, synth, dev, T, args.replicas, to_dev, side)

    if not args.no_cache:
        out["expert_cache"] = cache_bench(torch, seedmm, synth, host, P)

    if not args.no_encoder:
        out["encoder"] = encoder_bench(torch, seedmm, synth, P, args.no_cpu)

    if not args.no_cpu:
        import oracle
        s0 = args.warmup
        ids0 = ids_h[s0]
        x0 = synth.bf16_bits_to_f32(x_d[s0].view(torch.int16).cpu().numpy().view(np.uint16))
        w0 = w_d[s0].cpu().numpy()
        d0 = len(np.unique(ids0))

        def oracle_rate(budget_s, reps=5):
            """Median over `reps` runs of the oracle's time per token, each run a block of
            consecutive tokens of the step sized from a first token so that all runs
            together take about budget_s; returns (s per token, tokens per run)."""
            t0 = time.perf_counter()
            oracle.moe(ids0[:1], w0[:1], x0[:1], E, H, I, P, host["gate"], host["up"], host["down"])
            per = time.perf_counter() - t0
            n = int(max(1, min(T, budget_s / reps / max(per, 1e-9))))
            times = []
            for r_ in range(reps):
                a = (r_ * n) % max(T - n + 1, 1)
                t0 = time.perf_counter()
                oracle.moe(ids0[a:a + n], w0[a:a + n], x0[a:a + n], E, H, I, P,
                           host["gate"], host["up"], host["down"])
                times.append((time.perf_counter() - t0) / n)
            return float(np.median(times)), n, [float(v) for v in times]

        threads = oracle.num_threads()
        t_tok, n_tok, runs = oracle_rate(args.cpu_seconds)
        t_cpu = t_tok * T                      # the oracle's cost is linear in tokens
        oracle.set_num_threads(1)
        t_tok1, n_tok1, runs1 = oracle_rate(args.cpu_seconds / 3)
        oracle.set_num_threads(threads)
        t_cpu1 = t_tok1 * T
        out["cpu_baseline"] = {
            "value": d0 * 3 * w_per_mat / t_cpu, "unit": "weights/s",
            "cores": threads, "kind": "oracle",
            "sample": f"oracle MoE on blocks of {n_tok} consecutive tokens of one {T}-token step, "
                      f"median of {len(runs)} runs, scaled linearly to the step",
            "tok_s": T / t_cpu, "s_per_token_runs": runs,
            "single_thread": {"value": d0 * 3 * w_per_mat / t_cpu1, "tok_s": T / t_cpu1,
                              "sample": f"blocks of {n_tok1} tokens, one thread, median of "
                                        f"{len(runs1)} runs"},
            "host": host_cpu()}
        if not args.eager:
            # the timed configuration against the oracle: the first tokens of input set 0
            # as the graph replays computed them (two streams, replica 0 = these weights)
            ids_g, w_g = synth.route_topk(base, f"router.T{T}.s0", T, E, TOPK)
            x_g = synth.bf16_bits_to_f32(synth.bf16_bits(synth.normal_f32(base, f"x.T{T}.s0", (T, H))))
            npar = min(4, T)
            ref = oracle.moe(ids_g[:npar], w_g[:npar], x_g[:npar], E, H, I, P,
                             host["gate"], host["up"], host["down"])
            errs = [float(np.linalg.norm(y_graph0[t].astype(np.float64) - ref[t]) /
                          max(np.linalg.norm(ref[t]), 1e-300)) for t in range(npar)]
            out["parity"] = {"tokens": npar, "max_rel_l2": max(errs), "tolerance": 1e-2,
                             "ok": max(errs) <= 1e-2,
                             "path": "graph replay of the timed step, input set 0, replica 0"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
