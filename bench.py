"""Benchmark of the fused linear + cross-entropy path (forward + backward).

One step = lce_forward + lce_backward over one batch of seeded synthetic
input already resident in HBM: valid-token compaction, fused projection +
online logsumexp, chunk merge, loss reduction, dH zeroing of ignored rows,
operand layout for backward, logit recompute + G, dH += G W, dW += G^T H.

Default workload: the Llama-3-8B-shaped head (N = 4 x 2048 tokens, d = 4096,
V = 128256, per-sequence valid lengths uniform in [512, 2048], Zipf labels).
Prints one JSON line with valid tokens/s, TFLOP/s (8 N_valid d V per step),
the roofline entry of the dominant kernel (device time from HIP events on
the launch stream), and the fp64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "valid tokens/sec and % bf16 MFMA peak, fused linear-CE fwd+bwd, d=4096 V=128256"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0

# FLOPs per step of each kernel class, as a multiple of N_valid * d * V
CLASS_FLOPS = {"fwd": 2, "bwd_g": 2, "dh": 2, "dw": 2, "dh_dw": 4}


_CSRC = "vocab_cross_entropy_valid_amd/csrc/"
# Sources that determine each kernel class's device code: its own file, the
# shared device header, the argument structs and the build flags.
_SHARED_SOURCES = (_CSRC + "device_common.h", _CSRC + "kernels.h",
                   "vocab_cross_entropy_valid_amd/build.py")
KERNEL_FILE = {"compact": "kernels_fwd.hip", "fwd": "kernels_fwd.hip", "merge": "kernels_fwd.hip",
               "reduce": "kernels_fwd.hip", "zero": "kernels_bwd.hip",
               "transpose": "kernels_bwd.hip", "bwd_g": "kernels_bwd.hip", "dh": "kernels_bwd.hip",
               "dw": "kernels_bwd.hip", "gemm": "kernels_bwd.hip", "embed": "kernels_embed.hip",
               "attn": "kernels_attn.hip", "attn_dq": "kernels_attn.hip",
               "attn_dkv": "kernels_attn.hip", "dh_dw": "kernels_bwd.hip",
               "cast": "kernels_bwd.hip", "mfma": "kernels_bwd.hip", "opt": "kernels_bwd.hip"}


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest(kernel: str) -> str:
    """sha256 over the sources that determine one kernel class's device code."""
    import hashlib
    h = hashlib.sha256()
    for rel in (_CSRC + KERNEL_FILE[kernel],) + _SHARED_SOURCES:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary.

    The summary (profiles/hbm_traffic_<kernel>_kernel_<workload>.md) holds
    FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the same
    counter reads for a plain copy of known size, and the source digest of
    the kernels it was taken on.  Returns None when there is no summary or
    the kernels have changed since.
    """
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kernel}_kernel_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip().lstrip("- ").strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_digest(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(mib: int, dev) -> None:
    """A plain streaming copy of known size (reads and writes mib MiB), three times."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    _log(f"[bench] copy probe: 3 x {mib} MiB read + {mib} MiB written (elementwise kernel)")


def cpu_baseline(H, W, y, target_s: float):
    """The fp64 oracle on a sample of valid rows (full V and d), timed."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        threads = sum(p.get("num_threads", 0) for p in threadpoolctl.threadpool_info()
                      if p.get("user_api") == "blas") or None
    except Exception:  # noqa: BLE001
        threads = None
    cores = len(os.sched_getaffinity(0))
    valid = np.flatnonzero(y != -100)

    def run(nrows):
        rows = valid[:nrows]
        t0 = time.perf_counter()
        oracle.forward(H[rows], W, y[rows], -100)
        oracle.backward(H[rows], W, y[rows], -100)
        return time.perf_counter() - t0

    # t(n) = fixed (float64 copies of W) + n * per_row; fit from two sizes
    n1, n2 = 8, 32
    t1, t2 = run(n1), run(n2)
    per_row = max((t2 - t1) / (n2 - n1), 1e-6)
    fixed = max(t1 - n1 * per_row, 0.0)
    n = int(min(len(valid), max(n2, (target_s - fixed) / per_row)))
    t = run(n) if n > n2 else t2
    return {"value": n / t, "unit": "valid tokens/s", "cores": threads or cores,
            "kind": "oracle",
            "sample": f"{n} valid rows of the same workload (full V and d), fp64 forward + "
                      f"backward, {t:.1f} s; host cores available: {cores}"}


ATTN_METRIC = "online-softmax attention forward+backward TFLOP/s and % bf16 MFMA peak, causal, B=8 H=32 S=2048 D=128"


def attention_pairs(S: int, causal: bool) -> int:
    """(query, key) pairs the mask leaves: each costs 4 D FLOPs (QK^T and PV)."""
    return S * (S + 1) // 2 if causal else S * S


def cpu_baseline_attention(wl, Q, K, V, dO, target_s: float):
    """The fp64 attention oracle (forward + backward) on whole heads of the same workload."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    flops_head = ATTN_FLOPS_PER_PAIR * wl.D * attention_pairs(wl.S, wl.causal)
    t0 = time.perf_counter()
    heads = 0
    while heads < wl.B * wl.H:
        b, h = divmod(heads, wl.H)
        oracle.attention_forward(Q[b, h], K[b, h], V[b, h], causal=wl.causal)
        oracle.attention_backward(Q[b, h], K[b, h], V[b, h], dO[b, h], causal=wl.causal)
        heads += 1
        if time.perf_counter() - t0 >= target_s:
            break
    t = time.perf_counter() - t0
    return {"value": heads * flops_head / t / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{heads} of the {wl.B * wl.H} heads (S {wl.S}, D {wl.D}, causal), fp64 "
                      f"full-score softmax forward + backward, {t:.1f} s; host cores "
                      f"available: {cores}"}


# FLOPs per unmasked (query, key) pair, in units of D: forward S = Q K^T and
# O = P V (2 + 2); backward S recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K,
# dK = dS^T Q (2 each).  The backward's two passes execute S and dP twice:
# the dQ pass runs S, dP, dQ (6) and the dK / dV pass S, dP, dV, dK (8).
ATTN_FLOPS_PER_PAIR = 14
ATTN_KERNEL_FLOPS_PER_PAIR = {"attn": 4, "attn_dq": 6, "attn_dkv": 8}


def bench_attention(args) -> None:
    """Times lce_attention_forward + lce_attention_backward on the Llama-3-8B-shaped
    attention batch (one step = forward, then backward for a fixed upstream dO)."""
    import torch

    import workloads
    from vocab_cross_entropy_valid_amd import _lib, torch_api

    wl = workloads.ATTENTION
    _log(f"[bench] generating {wl.name}: B={wl.B} H={wl.H} S={wl.S} D={wl.D} causal={wl.causal}")
    Q, K, V = workloads.attention_inputs(wl.B, wl.H, wl.S, wl.D, wl.seed)
    dO = workloads.attention_inputs(wl.B, wl.H, wl.S, wl.D, wl.seed + 1000)[0]
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous() for x in (Q, K, V)]
    dOt = torch.from_numpy(dO).to(dev).to(torch.bfloat16).contiguous()
    f32 = dict(dtype=torch.float32, device=dev)
    shape = (wl.B, wl.H, wl.S, wl.D)
    out = torch_api.AttentionOut(O=torch.empty(*shape, **f32),
                                 lse=torch.empty(wl.B, wl.H, wl.S, **f32))
    grads = torch_api.AttentionGrads(dQ=torch.empty(*shape, **f32), dK=torch.empty(*shape, **f32),
                                     dV=torch.empty(*shape, **f32))
    delta = torch.empty(wl.B, wl.H, wl.S, **f32)

    def step():
        torch_api.attention_forward(*t, causal=wl.causal, out=out)
        torch_api.attention_backward(*t, out, dOt, causal=wl.causal, out=grads, delta=delta)

    torch.cuda.synchronize()
    # one step takes a few ms: the clock needs tens of launches to settle, so
    # the attention leg warms up with at least 20 steps (reported as "warmup")
    warmup = max(args.warmup, 20)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    _lib.lce_timing_reset()
    _lib.lce_timing_enable(True)
    _log(f"[bench] timing {args.steps} attention steps (forward + backward)")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.lce_timing_enable(False)
    pairs = attention_pairs(wl.S, wl.causal) * wl.B * wl.H
    kernels = {}
    for name, per_pair in ATTN_KERNEL_FLOPS_PER_PAIR.items():
        ms, n = _lib.lce_timing_query(_lib.KERNEL_CLASSES.index(name))
        avg_us = 1e3 * ms / max(n, 1)
        fl = per_pair * wl.D * pairs
        kernels[name] = {"ms_per_step": round(ms / args.steps, 4), "launches_per_step": n / args.steps,
                         "avg_launch_us": round(avg_us, 2), "flops_per_launch": fl,
                         "tflops": round(fl / (avg_us * 1e-6) / 1e12, 2)}
    _lib.lce_timing_reset()
    for x in (out.O, grads.dQ, grads.dK, grads.dV):
        assert bool(torch.isfinite(x).all())
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, dev)
    flops = ATTN_FLOPS_PER_PAIR * wl.D * pairs
    ms_step = 1e3 * elapsed / args.steps
    tflops = flops / (ms_step * 1e-3) / 1e12
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    kd = kernels[dom]
    res = {
        "metric": ATTN_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0, 1) Q, K, V and dO rounded to bf16 (no dataset)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "S": wl.S, "D": wl.D,
                   "causal": wl.causal},
        "pct_peak_bf16": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "positions_per_s": round(wl.B * wl.S / (ms_step * 1e-3), 1),
        "score_matrix_bytes_avoided": 4 * wl.B * wl.H * wl.S * wl.S,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": kd["tflops"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kd["tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": counter_traffic(dom, wl.name),
                     "flops_per_launch": kd["flops_per_launch"],
                     "avg_launch_us": kd["avg_launch_us"]},
        "kernels": kernels,
    }
    if args.cpu_seconds > 0:
        _log("[bench] timing the CPU attention oracle on whole heads")
        res["cpu_baseline"] = cpu_baseline_attention(wl, Q, K, V, dO, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_mfma_probe(args) -> None:
    """lce_mfma_peak: the bf16 MFMA rate with register operands and no memory
    traffic (the chip's own ceiling for the matrix cores, to set the path's
    kernels against; under a counter run it also gives the clock)."""
    import torch

    from vocab_cross_entropy_valid_amd import _lib
    dev = torch.device("cuda:0")
    n_out, iters = 1024 * 512, 20000
    out = torch.empty(n_out, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        _lib.lce_mfma_peak(out.data_ptr(), n_out, iters, s)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        _lib.lce_mfma_peak(out.data_ptr(), n_out, iters, s)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 1024 * 8 * 4 * iters * 32768.0
    tf = flops / (ms * 1e-3) / 1e12
    assert bool(torch.isfinite(out).all())
    print(json.dumps({"metric": "bf16 MFMA rate, register operands, no memory traffic",
                      "value": round(tf, 1), "unit": "TFLOP/s", "n_gpus": 1, "ms_per_launch":
                      round(ms, 3), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                      "peak": PEAK_BF16_TFLOPS}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the CPU oracle sample (0 disables it)")
    ap.add_argument("--no-gemm", action="store_true", help="skip the bare-GEMM reference rate")
    ap.add_argument("--shards", type=int, default=1,
                    help="split the vocabulary into this many contiguous shards: each step runs "
                         "the shard forwards, the merge and the shard backwards")
    ap.add_argument("--fused-opt", choices=["sgd", "adamw"], default=None,
                    help="backward with the optimizer applied in the dW epilogue (no dW table); "
                         "fp32 master weights and AdamW state are allocated")
    ap.add_argument("--tied-input", action="store_true",
                    help="also run the input side of a tied table each step: the masked "
                         "embedding gather of the shifted labels and the scatter-sum of a "
                         "synthetic dX into dW")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run a plain device copy of this many MiB "
                         "three times (calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--attention", action="store_true",
                    help="measure online-softmax attention (batch 8 x 32 heads x 2048 x 128, "
                         "causal) instead of the loss path")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="measure the pure bf16 MFMA rate (register operands, no memory "
                         "traffic) instead of the loss path")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(token rows would shard across GPUs, with no communication in the "
              "forward; the vocabulary-shard entry points cover a split table)",
              file=sys.stderr)
        sys.exit(2)

    if args.attention:
        bench_attention(args)
        return
    if args.mfma_probe:
        bench_mfma_probe(args)
        return

    import numpy as np
    import torch

    import workloads
    from vocab_cross_entropy_valid_amd import _lib, torch_api

    wl = workloads.CONFIGS[args.config]
    _log(f"[bench] generating {wl.name}: N={wl.N} d={wl.d} V={wl.V} {wl.dtype}")
    H, W, y = workloads.generate(args.config)
    n_valid = int(np.count_nonzero(y != -100))
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    Ht = torch.from_numpy(H).to(dev, dt)
    Wt = torch.from_numpy(W).to(dev, dt)
    yt = torch.from_numpy(y).to(dev)
    dH = torch.empty(wl.N, wl.d, dtype=torch.float32, device=dev)
    dW = torch.empty(wl.V, wl.d, dtype=torch.float32, device=dev)
    g = torch.ones(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    ws = torch_api.alloc_workspace(wl.N, wl.d, wl.V, dt, dev, step=bool(args.fused_opt))

    def step():
        fwd = torch_api.forward(Ht, Wt, yt, workspace=ws, check=False)
        torch_api.backward(Ht, Wt, yt, fwd, grad_out=g, dH=dH, dW=dW, workspace=ws)
        return fwd

    if args.shards > 1:
        # contiguous shards of (nearly) equal size; W slices are views of one table
        K = args.shards
        edges = [round(k * wl.V / K) for k in range(K + 1)]
        shards = [(edges[k], edges[k + 1]) for k in range(K)]
        Wsh = [Wt[a:b] for a, b in shards]
        dWsh = [dW[a:b] for a, b in shards]
        wss = torch_api.alloc_workspace(wl.N, wl.d, max(b - a for a, b in shards), dt, dev)
        pm = torch.empty(K, wl.N, dtype=torch.float32, device=dev)
        ps, pt = torch.empty_like(pm), torch.empty_like(pm)
        vidx = torch.empty(wl.N, dtype=torch.int32, device=dev)
        vcnt = torch.empty(1, dtype=torch.int32, device=dev)
        errf = torch.empty(1, dtype=torch.int32, device=dev)
        parts = [torch_api.ShardPartials(pm[k], ps[k], pt[k], vidx, vcnt, errf)
                 for k in range(K)]

        def step():  # noqa: F811
            for k, (a, b) in enumerate(shards):
                torch_api.forward_shard(Ht, Wsh[k], yt, wl.V, a, workspace=wss, out=parts[k])
            fwd = torch_api.lse_merge(pm, ps, pt, vidx, vcnt)
            for k, (a, b) in enumerate(shards):
                torch_api.backward_shard(Ht, Wsh[k], yt, wl.V, a, fwd, dH, accumulate_dH=k > 0,
                                         grad_out=g, dW_shard=dWsh[k], workspace=wss)
            return fwd

    fused = None
    if args.fused_opt:
        if args.tied_input or args.shards > 1:
            print("--fused-opt runs alone (not with --tied-input or --shards)", file=sys.stderr)
            sys.exit(2)
        master = Wt.float()
        ea = torch.zeros_like(master) if args.fused_opt == "adamw" else None
        eas = torch.zeros_like(master) if args.fused_opt == "adamw" else None
        del dW
        dW = None
        fused = {"optimizer": args.fused_opt, "state_bytes": master.numel() * 4 *
                 (3 if args.fused_opt == "adamw" else 1), "dW_table_bytes_avoided": wl.V * wl.d * 4}
        t_step = [0]

        def step():  # noqa: F811
            t_step[0] += 1
            fwd = torch_api.forward(Ht, Wt, yt, workspace=ws, check=False)
            torch_api.backward_step(Ht, Wt, yt, fwd, args.fused_opt, 1e-6, 0.0, step=t_step[0],
                                    W_master=master, exp_avg=ea, exp_avg_sq=eas, grad_out=g,
                                    dH=dH, workspace=ws)
            return fwd

    tied = None
    if args.tied_input:
        # next-token inputs: position n reads the previous position's label; the
        # first position and the padded ones read the padding id -1
        ids = np.concatenate([[-1], y[:-1]]).astype(np.int64)
        ids[ids == -100] = -1
        idt = torch.from_numpy(ids).to(dev)
        dXt = torch.randn(wl.N, wl.d, dtype=torch.float32, device=dev)
        ews = torch.empty(_lib.lce_embed_workspace_bytes(wl.N, wl.d, wl.V), dtype=torch.uint8,
                          device=dev)
        n_in = int(np.count_nonzero(ids != -1))
        uniq = int(np.unique(ids[ids != -1]).size)
        esz = 2 if wl.dtype == "bf16" else 4
        tied = {"pad_id": -1, "valid_inputs": n_in, "distinct_ids": uniq,
                # gather: valid rows of W read, every row of X written; backward: valid
                # rows of dX read, each touched dW row read and written
                "algorithmic_bytes": n_in * wl.d * esz + wl.N * wl.d * esz
                + n_in * wl.d * 4 + 2 * uniq * wl.d * 4}
        base_step = step

        def step():  # noqa: F811
            emb = torch_api.embed_forward(Wt, idt, -1)
            fwd = base_step()
            torch_api.embed_backward(dXt, idt, emb, dW, accumulate_dW=True, workspace=ews)
            return fwd

    # Peak device memory of one step beyond everything held before it (inputs,
    # gradient outputs, optimizer state) and the per-token forward outputs it
    # allocates (loss, lse, index, count, sums, flag): the scratch the step
    # needs, which must be the workspace the library asks for and nothing
    # else.  Measured for the plain and the fused-update step.
    ws_measured = None
    if args.shards == 1 and not args.tied_input:
        torch.cuda.synchronize()
        mem_base = torch.cuda.memory_stats(dev)["requested_bytes.all.current"] - ws.numel()
        torch.cuda.reset_peak_memory_stats(dev)
        fwd = step()
        torch.cuda.synchronize()
        fwd_out = sum(t.numel() * t.element_size() for t in
                      (fwd.loss, fwd.lse, fwd.valid_idx, fwd.valid_count, fwd.loss_sum,
                       fwd.loss_mean, fwd.err_flag))
        ws_measured = int(torch.cuda.memory_stats(dev)["requested_bytes.all.peak"] - mem_base
                          - fwd_out)
        del fwd

    _log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        fwd = step()
    torch.cuda.synchronize()
    _lib.lce_check_error(fwd.err_flag.data_ptr(), torch.cuda.current_stream().cuda_stream)

    _lib.lce_timing_reset()
    _lib.lce_timing_enable(True)
    _log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd = step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.lce_timing_enable(False)
    kernels = {}
    for k, name in enumerate(_lib.KERNEL_CLASSES):
        ms, n = _lib.lce_timing_query(k)
        if n:
            kernels[name] = {"ms_per_step": ms / args.steps, "launches_per_step": n / args.steps,
                             "avg_launch_us": 1e3 * ms / n}
    _lib.lce_timing_reset()
    # the same steps again without the per-launch events: each launch is
    # bracketed by two event records in the timed region above, which costs
    # ~2% of a step; this figure is context, the headline stays the timed one
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd = step()
    torch.cuda.synchronize()
    ms_plain = 1e3 * (time.perf_counter() - t0) / args.steps
    assert int(fwd.valid_count.item()) == n_valid
    loss_mean = float(fwd.loss_mean.item())
    _log(f"[bench] done: {1e3 * elapsed / args.steps:.3f} ms/step, mean loss {loss_mean:.5f}")

    ms_step = 1e3 * elapsed / args.steps
    flops = 8.0 * n_valid * wl.d * wl.V
    tflops = flops / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS

    # roofline entry of the dominant kernel class (largest device time per step)
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    if dom in CLASS_FLOPS:
        per_step = CLASS_FLOPS[dom] * n_valid * wl.d * wl.V
        ach = per_step / (kernels[dom]["ms_per_step"] * 1e-3) / 1e12
        traffic = counter_traffic(dom, wl.name)
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                    "traffic": None if traffic is None else round(traffic),
                    "flops_per_launch": per_step / kernels[dom]["launches_per_step"],
                    "avg_launch_us": round(kernels[dom]["avg_launch_us"], 2)}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": None, "traffic": None}

    # HBM / latency passes: algorithmic bytes per step and the rate they reach
    esz = 2 if wl.dtype == "bf16" else 4
    n_vt = -(-wl.V // 256)
    tpc = max(1, -(-n_vt // 64))
    J = -(-n_vt // tpc)  # vocabulary chunks of the forward (as the library plans them)
    pass_bytes = {
        # labels read; index, count and flag written; loss and lse zeroed on ignored rows
        "compact": 8 * wl.N + 4 * n_valid + 8 + 8 * (wl.N - n_valid),
        # (max, sum, target) partials of every chunk read, index and label read,
        # lse, loss and the compact loss written
        "merge": 12 * J * n_valid + 12 * n_valid + 12 * n_valid,
        "reduce": 4 * n_valid + 16,
        # fp32 dH rows of ignored tokens zeroed, labels read
        "zero": 4 * (wl.N - n_valid) * wl.d + 8 * wl.N,
        # H^T of the valid rows, read and written (once per token chunk; the
        # fused update walks vocabulary blocks outside and rebuilds it per
        # block); W^T of every vocabulary block too where dH cannot read W
        # directly (fp32, fused update)
        "transpose": 2 * esz * wl.d * (n_valid * (-(-wl.V // 16384) if args.fused_opt else 1)
                                       + (0 if wl.dtype == "bf16" and not args.fused_opt
                                          else wl.V)),
    }
    hbm_passes = {}
    for name, nbytes in pass_bytes.items():
        if name in kernels:
            gbs = nbytes / (kernels[name]["ms_per_step"] * 1e-3) / 1e9
            hbm_passes[name] = {"bytes_per_step": int(nbytes), "GB/s": round(gbs, 1),
                                "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}

    if tied is not None and "embed" in kernels:
        k = kernels["embed"]
        tied["embed_ms_per_step"] = round(k["ms_per_step"], 4)
        tied["GB/s"] = round(tied["algorithmic_bytes"] / (k["ms_per_step"] * 1e-3) / 1e9, 1)
        tied["peak_GB/s"] = PEAK_HBM_GBS

    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, dev)

    gemm = None
    if not args.no_gemm and wl.dtype == "bf16":
        # bare GEMM of the same engine at the forward's shape (N_valid x V x d)
        A = Ht[:n_valid].contiguous()
        C = torch.empty(n_valid, wl.V, dtype=torch.float32, device=dev)
        s = torch.cuda.current_stream().cuda_stream
        for _ in range(2):
            _lib.lce_gemm_nt(A.data_ptr(), Wt.data_ptr(), C.data_ptr(), n_valid, wl.V, wl.d,
                             _lib.LCE_BF16, s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        reps = 5
        for _ in range(reps):
            _lib.lce_gemm_nt(A.data_ptr(), Wt.data_ptr(), C.data_ptr(), n_valid, wl.V, wl.d,
                             _lib.LCE_BF16, s)
        e1.record()
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / reps
        gemm = {"shape": [n_valid, wl.V, wl.d], "ms": round(gms, 3),
                "tflops": round(2.0 * n_valid * wl.V * wl.d / (gms * 1e-3) / 1e12, 1)}
        del C
        # the vendor library's bare GEMM at the same shape (torch's Linear path,
        # bf16 in and out, fp32 accumulation): context for the fused kernels'
        # rate, outside the timed steps
        F = torch.nn.functional
        for _ in range(2):
            Cv = F.linear(A, Wt)
        e0.record()
        for _ in range(reps):
            Cv = F.linear(A, Wt)
        e1.record()
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / reps
        gemm["vendor_linear_ms"] = round(vms, 3)
        gemm["vendor_linear_tflops"] = round(2.0 * n_valid * wl.V * wl.d / (vms * 1e-3) / 1e12, 1)
        del Cv

    cpu = None
    if args.cpu_seconds > 0:
        _log("[bench] timing the CPU oracle on a sample")
        cpu = cpu_baseline(H, W, y, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(n_valid / (ms_step * 1e-3), 1),
        "unit": "valid tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: seeded Gaussian H, W and Zipf labels with padding (no dataset)",
        "config": {"workload": wl.name + (f" in {args.shards} vocabulary shards"
                                          if args.shards > 1 else "")
                   + (" with the tied input side" if args.tied_input else "")
                   + (f" with {args.fused_opt} fused into dW" if args.fused_opt else ""), "N": wl.N, "d": wl.d, "V": wl.V,
                   "N_valid": n_valid, "ignore_index": -100, "seed": wl.seed},
        "tflops": round(tflops, 2),
        "pct_peak_bf16": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "mean_loss": loss_mean,
        # measured: peak of one step minus inputs and outputs; planned: the
        # library's lce_(step_)workspace_bytes for these sizes
        "workspace_bytes": ws_measured,
        "workspace_bytes_planned": int(ws.numel()),
        "logits_table_bytes_avoided": wl.N * wl.V * 4,
        "roofline": roofline,
        "ms_per_step_without_events": round(ms_plain, 4),
        "value_without_events": round(n_valid / (ms_plain * 1e-3), 1),
        "hbm_passes": hbm_passes,
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kernels.items()},
        "gemm_engine_reference": gemm,
        "tied_input": tied,
        "fused_optimizer": fused,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
