"""Throughput of one POET-X layer training step (forward + backward) on one
MI355X, through libpoetx.so.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config square]
                    [--cpu-sample-tokens N | --no-cpu]

A step is the whole hot path on one batch of synthetic tokens: Cayley-Neumann
forward for both sides, the input-centric forward pass, the backward pass, and
the Cayley-Neumann backward for both sides.  The permutation fold happens once
before timing (once per inner loop).  Inputs are resident in HBM when timing
starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "POET-X layer fwd+bwd tokens/s at 4096², b=256; % MFMA peak; CNP blocks/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0


def step_flops(cfg) -> float:
    """Algorithmic flops of one step: 4mn + 6b(m+n) per token (Z and dV
    products, the four per-token block products forward and backward, and the
    two block reductions) plus 6 k b^2 (m+n) for the Cayley-Neumann passes."""
    m, n, b, k, T = cfg.m, cfg.n, cfg.b, cfg.k, cfg.T
    return T * (4.0 * m * n + 6.0 * b * (m + n)) + 6.0 * k * b * b * (m + n)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="square")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--xmem", action="store_true",
                    help="memory-saving mode: keep only U, recompute Z in the backward")
    ap.add_argument("--xq", action="store_true",
                    help="int8 base weight (per-row scales), expanded to bf16 in each pass")
    ap.add_argument("--keep-w0ft", action="store_true",
                    help="also keep the folded weight transposed and let the backward's dense "
                         "product read that copy instead of W0f itself (same results)")
    ap.add_argument("--fused-gather", action="store_true",
                    help="run each input-side gather and the block products after it as one "
                         "pass (bf16, b = 256, gathered width up to 4096) instead of a gather "
                         "pass and a block pass")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel of each timed step from the host instead of "
                         "replaying one captured HIP graph of the step")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run a plain 1 GiB elementwise copy "
                         "(torch.neg) three times: the reference kernel that calibrates "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer "
              "would shard over tokens with one all-reduce of the packed gradients; that "
              "multi-GPU path is not implemented)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from orthogonal_reparameterized_02_amd import inputs as I
    from orthogonal_reparameterized_02_amd import poetx as P
    from orthogonal_reparameterized_02_amd._lib import lib
    from orthogonal_reparameterized_02_amd.layer import POETXLayer

    cfg = I.CONFIG_BY_NAME[args.config]
    act = P.BF16 if cfg.dtype == "bf16" else P.F32
    torch.cuda.set_device(0)
    d = I.make_inputs(cfg, seed=args.seed, f64=False)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    P.poetx_set_fused_gather(args.fused_gather)  # before the workspaces are sized
    L = POETXLayer(cfg.m, cfg.n, cfg.b, cfg.k, cfg.T, act, xmem=args.xmem, xq=args.xq,
                   keep_w0ft=args.keep_w0ft)
    if args.xq:
        q, sc = I.quantize_rows_int8(I.make_inputs(cfg, seed=args.seed, want=("W0",))["W064"])
        L.load_q(torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda(), dev(d["theta_P"]),
                 dev(d["theta_R"]), dev(d["perm_P"]), dev(d["perm_R"]))
    else:
        L.load(dev(d["W0"]), dev(d["theta_P"]), dev(d["theta_R"]), dev(d["perm_P"]),
               dev(d["perm_R"]))
    x, dy = dev(d["x"]), dev(d["dy"])
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        L.step(x, dy)
    torch.cuda.synchronize()

    # The step has a fixed shape and fixed buffers, so it is captured once as
    # a HIP graph (15 kernels, no memsets) and replayed: the same kernels on
    # the same data, without a host launch per kernel.  --eager launches them.
    if args.eager:
        run_step = lambda: L.step(x, dy)  # noqa: E731
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            L.step(x, dy)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run_step = graph.replay

    # ---- timed region: exactly K steps -----------------------------------
    # (an event between consecutive steps as well, for the per-step spread)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        run_step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])

    # ---- per-stage times: the same K steps again with boundary events ----
    # (events are recorded on the stream the kernels run on)
    nev = 8
    fwd_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    bwd_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    cnp_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for evs in fwd_ev + bwd_ev:      # torch creates the HIP events on first record
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()
    import ctypes as C

    def hook(evs):
        arr = (C.c_void_p * nev)(*[e.cuda_event for e in evs])
        rc = lib().poetx_set_stage_events(C.cast(arr, C.c_void_p), nev)
        assert rc == 0, lib().poetx_last_error()

    for s in range(args.steps):
        cnp_ev[s][0].record(stream)
        L.cnp()
        cnp_ev[s][1].record(stream)
        hook(fwd_ev[s])
        L.layer_fwd(x)
        hook(bwd_ev[s])
        L.layer_bwd(dy)
        lib().poetx_set_stage_events(None, 0)
        cnp_ev[s][2].record(stream)
        L.cnp_bwd()
        cnp_ev[s][3].record(stream)
    torch.cuda.synchronize()

    def mean_ms(evs, i, j):
        return float(np.mean([e[i].elapsed_time(e[j]) for e in evs]))

    # (with --fused-gather, gather_x and gather_dy hold the one-pass kernel and
    # blocks_P, blocks_R_bwd only the event gap)
    fwd_names = ["gather_x", "blocks_P", "dense_Z", "blocks_R", "scatter_y"]
    bwd_names = ["gather_dy", "blocks_R_bwd", "dG_R", "dense_dV", "blocks_P_bwd", "dG_P", "scatter_dx"]
    stages = {nm: mean_ms(fwd_ev, i, i + 1) * 1e3 for i, nm in enumerate(fwd_names)}
    stages.update({nm: mean_ms(bwd_ev, i, i + 1) * 1e3 for i, nm in enumerate(bwd_names)})
    stages["cnp_fwd"] = mean_ms(cnp_ev, 0, 1) * 1e3
    stages["cnp_bwd"] = mean_ms(cnp_ev, 2, 3) * 1e3

    # ---- once per inner loop (not part of the step): merge W0 <- R W0 P ----
    # (an int8 base weight has no bf16 copy to merge into)
    merge_us = None
    if not args.xq:
        merge_ws = torch.empty(P.poetx_workspace_bytes(L.sh, 4), dtype=torch.uint8, device="cuda")
        merged = torch.empty(cfg.m, cfg.n, dtype=L.dtype, device="cuda")
        mev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for i in range(6):
            if i == 1:
                mev[0].record(stream)
            P.poetx_merge(L.sh, L.W0f, L.G_R, L.GT_P, L.perm_R_inv, L.perm_P_inv, merged,
                          merge_ws)
        mev[1].record(stream)
        torch.cuda.synchronize()
        merge_us = round(mev[0].elapsed_time(mev[1]) / 5 * 1e3, 2)
        del merge_ws, merged

    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    T, m, n, b = cfg.T, cfg.m, cfg.n, cfg.b
    flops = step_flops(cfg)
    peak = PEAK_BF16_TFLOPS if act == P.BF16 else PEAK_FP32_TFLOPS
    tokens_per_s = T / (ms * 1e-3)
    # The roofline covers both dense launches of the step (the forward
    # Z = V W0f^T and the backward dV = dZ W0f), as the rocprofv3 average of
    # the kernel does.  b = 256 or 128 in bf16: each also forms its block
    # product in the epilogue (S = Z G_R^T, dU = dV G_P: 2 m b and 2 n b
    # flops per token more), where the output width is a multiple of 256.
    fused_f = act == P.BF16 and b in (128, 256) and m % 256 == 0
    fused_b = act == P.BF16 and b in (128, 256) and n % 256 == 0
    fused = fused_f and fused_b
    flops_pair = (2.0 * T * m * n + (2.0 * T * m * b if fused_f else 0.0)
                  + 2.0 * T * m * n + (2.0 * T * n * b if fused_b else 0.0))
    dense_us = (stages["dense_Z"] + stages["dense_dV"]) / 2
    dense_flops = flops_pair / 2
    dense_tflops = dense_flops / (dense_us * 1e-6) / 1e12
    nblocks = cfg.n_P + cfg.n_R

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if act == P.BF16 else "f32",
        "data": "synthetic (seeded Gaussian activations and weights, random permutations)",
        "config": {"workload": f"{cfg.name}: POET-X layer m={m} n={n} b={b} k={cfg.k} "
                               f"T={T} tokens, {cfg.dtype} activations/W0, fp32 theta"
                               + (", xmem (Z recomputed in the backward)" if args.xmem else "")
                               + (", xq (int8 base weight)" if args.xq else "")
                               + (", W0f kept transposed too" if args.keep_w0ft else "")
                               + (", one-pass gather + block products" if args.fused_gather
                                  else ""),
                   "m": m, "n": n, "b": b, "k": cfg.k, "tokens": T, "seed": args.seed},
        "mfma_peak_frac": flops / (ms * 1e-3) / (peak * 1e12),
        "step_tflops": flops / (ms * 1e-3) / 1e12,
        "cnp_blocks_per_s": {"fwd": nblocks / (stages["cnp_fwd"] * 1e-6),
                             "fwd_bwd": nblocks / ((stages["cnp_fwd"] + stages["cnp_bwd"]) * 1e-6)},
        "stages_us": {k: round(v, 2) for k, v in stages.items()},
        "inner_loop_merge_us": merge_us,
        "roofline": {"kernel": (f"k_nt4<{1 if b == 256 else 2}>"
                                + (" on the int8 weight (dequantized in the kernel)" if args.xq else "")
                                + ", both launches of the step: "
                                "Z = V W0f^T with S = Z G_R^T and dV = dZ W0f with dU = dV G_P "
                                "in the epilogue" if fused else
                                f"{unfused_dense_kernel(T, m)}, both launches of the step: "
                                "Z = V W0f^T and dV = dZ W0f"),
                     "bound": "mfma", "achieved": dense_tflops, "peak": peak,
                     "unit": "TFLOP/s", "frac": dense_tflops / peak,
                     # the committed counters are the bf16 kernel's: none for the int8 one
                     "traffic": measured_traffic(cfg.name) if fused and not args.xq else None,
                     "flops_per_launch": dense_flops, "avg_launch_us": dense_us},
        "wall_s_timed": wall,
        "launch": "eager" if args.eager else "hip_graph",
    }

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, args.seed, min(args.cpu_sample_tokens, T))
    print(json.dumps(out), flush=True)
    return 0


COPY_PROBE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_nt4_block_square_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "orthogonal_reparameterized_02_amd", "csrc", "gemm_mfma.hip")


def unfused_dense_kernel(T, m):
    """The kernel the library picks for the unfused Z = V W0f^T (T x m output):
    the 256 x 256 one from half a tile per CU up, the 256 x 128 one below."""
    tiles = -(-T // 256) * -(-m // 256)
    return "k_nt4<0>" if m % 256 == 0 and tiles >= 128 else "k_gemm_nt"


def measured_traffic(config_name: str):
    """HBM bytes per launch of the dense kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when that summary is absent, was
    taken on another workload, or the kernel source has changed since."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            fields = dict(line.split(":", 1) for line in f if line.startswith("- ") and ":" in line)
        fields = {k[2:].strip(): v.strip().strip("`") for k, v in fields.items()}
        with open(KERNEL_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if fields.get("source_sha256") != sha or fields.get("workload") != config_name:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(cfg, seed: int, ts: int, reps: int = 3, warmup: int = 1) -> dict:
    """The float64 oracle, as it stands, on the first `ts` tokens of the same
    workload: forward and backward (weights formed, CNP both sides), `warmup`
    untimed passes and then the median of `reps` timed ones.  Reports the
    BLAS library and the threads it ran with."""
    import numpy as np
    blas, cores = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api', '?')} {libs[0].get('version', '')}".strip()
            cores = max(i.get("num_threads", 1) for i in libs)
    except Exception:  # pragma: no cover
        pass
    import oracle as O
    from orthogonal_reparameterized_02_amd import inputs as I
    d = I.make_inputs(cfg, seed=seed, T=ts)

    def one_pass():
        O.layer_fwd(d["x64"], d["W064"], d["theta_P64"], d["theta_R64"], d["perm_P"],
                    d["perm_R"], cfg.b, cfg.k)
        O.layer_bwd(d["x64"], d["dy64"], d["W064"], d["theta_P64"], d["theta_R64"],
                    d["perm_P"], d["perm_R"], cfg.b, cfg.k)

    for _ in range(warmup):
        one_pass()
    times = []
    for _ in range(reps):
        t = time.perf_counter()
        one_pass()
        times.append(time.perf_counter() - t)
    med = float(np.median(times))
    return {"value": ts / med, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "blas": blas,
            "sample": f"first {ts} of {cfg.T} tokens of the same layer, forward+backward in "
                      f"float64 NumPy: {warmup} warm-up pass, median of {reps} timed passes "
                      f"({', '.join(f'{t:.2f}' for t in times)} s)"}


if __name__ == "__main__":
    sys.exit(main())
