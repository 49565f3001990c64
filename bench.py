"""Benchmark: one MuonClip layer step on one MI355X.

A step is the whole path on the MuonClip attention layer (hidden 7168,
64 heads x 128, batch 4 x seq 4096, bf16): the per-head causal max-logit
statistic on the forward's Q and K, the Muon step (momentum + Nesterov +
Frobenius pass, 5 quintic Newton-Schulz iterations as bf16 MFMA GEMMs,
scaled and decayed parameter write) on W_q, W_k, W_v [8192 x 7168] and
W_o [7168 x 8192], then the per-head W_q / W_k rescale at tau = 100.

Inputs are seeded and synthetic and resident in HBM before timing.  Per-kernel
times come from HIP events recorded by the library around each launch on the
benchmark stream.  The CPU baseline times the fp64 oracle on a bounded sample
of the same workload and extrapolates to one step.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense bf16
# a register-only MFMA loop measured on the box: 2.11-2.14 PFLOP/s, shader clock
# 2.07-2.10 GHz under that load
MFMA_BF16_MEASURED_TFLOPS = 2120.0
HBM_PEAK_GBS = 8000.0
MFMA_FP32_PEAK_TFLOPS = 157.3    # dense fp32 MFMA, the spec figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the readings of the 24-layer decoder and the MoE stack")
    ap.add_argument("--seed", type=int, default=5000)
    ap.add_argument("--blas-reference", action="store_true",
                    help="time torch.matmul (hipBLASLt) on the full, unsymmetric Newton-Schulz "
                         "products of the same shapes, for comparison, and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (to scale HBM counters)")
    return ap.parse_args()


def measured_traffic():
    """Per-launch HBM bytes from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, keyed by kernel; an entry is used only while the hash of its
    kernel source still matches the source the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "muonclip_layer_step_hbm_traffic.txt")
    if not os.path.exists(path):
        return {}
    data = {}
    for line in open(path):
        if line.startswith("TRAFFIC_JSON "):
            data = json.loads(line[len("TRAFFIC_JSON "):])
    out = {}
    for k, v in data.items():
        src = v.get("source")
        if not src or not os.path.exists(os.path.join(ROOT, src)):
            continue
        h = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()[:16]
        if h == v.get("source_sha256_16"):
            out[k] = v["total_bytes"]
    return out


def ns_flops(m, n):
    """Algorithmic flops of one Newton-Schulz iteration on a wide m x n matrix
    with the symmetric products counted once: X X^T (upper triangle incl.
    diagonal: m(m+1)/2 dots of length n), A A^T (m(m+1)/2 dots of length m),
    B X (m n dots of length m)."""
    return {"ns_syrk_xxt": m * (m + 1) * n, "ns_syrk_poly": m * m * (m + 1), "ns_gemm_bx": 2 * m * m * n}


def note(msg):
    """A progress line on stderr (the JSON result alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        print(json.dumps({"copy_calibration_bytes": src.numel(), "copies": 3,
                          "copy_GBs_read_plus_write": round(2 * src.numel() / ms / 1e6, 1)}))
        return

    if args.blas_reference:
        print(json.dumps(blas_reference(torch)), flush=True)
        return

    import matrix_orthogonalizing_optimizer_muon_amd as mm
    from synthetic import generators as gen

    dev = torch.device("cuda:0")
    wl = gen.workload(5)
    ex = wl.extra
    B, T, H, D, dm = ex["batch"], ex["seq"], ex["heads"], ex["d_head"], ex["d_model"]
    seed = args.seed

    # ---------------- inputs (not timed)
    qk = gen.qk_inputs_torch(seed, B, T, H, D, dm, ex["n_designated"], ex["targets"], dev)
    Wqkv = gen.bulk_normal_torch((3, H * D, dm), wl.weight_std, seed + 10, dev, torch.bfloat16)
    Wqkv[0].copy_(qk["Wq"])
    Wqkv[1].copy_(qk["Wk"])
    Wo = gen.bulk_normal_torch((1, dm, H * D), wl.weight_std, seed + 11, dev, torch.bfloat16)
    Gqkv = gen.bulk_normal_torch((3, H * D, dm), 1.0, seed + 12, dev, torch.bfloat16)
    Go = gen.bulk_normal_torch((1, dm, H * D), 1.0, seed + 13, dev, torch.bfloat16)
    Mqkv = gen.bulk_normal_torch((3, H * D, dm), 0.5, seed + 14, dev, torch.float32)
    Mo = gen.bulk_normal_torch((1, dm, H * D), 0.5, seed + 15, dev, torch.float32)
    # the forward's projections on the pre-update weights (model work, not timed)
    Q = (qk["X"] @ Wqkv[0].t()).view(B, T, H, D).contiguous()
    K = (qk["X"] @ Wqkv[1].t()).view(B, T, H, D).contiguous()
    del qk
    groups = [(Wqkv, Gqkv, Mqkv), (Wo, Go, Mo)]
    hp = mm.HParams(lr=wl.lr, momentum=wl.momentum, weight_decay=wl.weight_decay,
                    nesterov=True, ns_steps=wl.ns_steps, ns_coeffs=wl.ns_coeffs,
                    ns_eps=wl.ns_eps, rms_target=wl.rms_target)
    ws = torch.empty(mm.workspace_size(groups), dtype=torch.uint8, device=dev)
    s_max = torch.empty(H, dtype=torch.float32, device=dev)
    clipped = torch.empty(H, dtype=torch.int32, device=dev)
    rm_ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        mm.qkclip_rowmax(Q, K, 1.0 / math.sqrt(D), True, out=s_max, workspace=rm_ws)
        mm.muon_step(groups, hp, workspace=ws)
        mm.qkclip_rescale(Wqkv[0], Wqkv[1], s_max, D, ex["tau"], ex["alpha"], clipped=clipped)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---------------- timed region
    mm.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = mm.profile_collect()
    mm.profile_enable(False)

    n_clipped = int((clipped == 1).sum())
    ms_per_step = 1e3 * elapsed / args.steps
    steps_per_s = args.steps / elapsed

    # ---------------- Newton-Schulz throughput and the dominant kernel's roofline
    m, n = 7168, 8192                      # every matrix is 7168 x 8192 once oriented wide
    n_mats = 4
    per_iter = ns_flops(m, n)
    ns_flop_step = n_mats * wl.ns_steps * sum(per_iter.values())
    # a symmetric product whose last wave is split runs as two kernels: the
    # whole tiles, then the last tiles' column halves (kind "<product>_slices")
    product_ms = {k: prof[k][0] + prof.get(k + "_slices", (0.0, 0))[0] for k in per_iter}
    ns_ms_step = sum(product_ms.values()) / args.steps
    ns_tflops = ns_flop_step / (ns_ms_step * 1e-3) / 1e12
    kernels = {k: {"total_ms": round(v[0], 4), "launches": v[1],
                   "avg_us": round(1e3 * v[0] / v[1], 2) if v[1] else None}
               for k, v in prof.items() if v[1]}
    dom = max(per_iter, key=lambda k: product_ms[k])
    dom_avg_s = product_ms[dom] / prof[dom][1] * 1e-3
    dom_flop = n_mats * per_iter[dom]
    achieved = dom_flop / dom_avg_s / 1e12
    traffic = measured_traffic()
    roofline = {"kernel": dom + (" + slices" if prof.get(dom + "_slices", (0.0, 0))[1] else ""), "bound": "mfma", "achieved": round(achieved, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": round(traffic[dom]) if dom in traffic else None,
                "measured_peak": MFMA_BF16_MEASURED_TFLOPS,
                "frac_of_measured_peak": round(achieved / MFMA_BF16_MEASURED_TFLOPS, 4)}

    # HBM passes: algorithmic bytes per launch over their event time
    elem = 4 * m * n
    hbm = {}
    mom_bytes = elem * (2 + 4 + 4 + 2 + 2)      # G bf16, M r/w fp32, X0 and X0^T bf16
    upd_bytes = elem * (2 + 2 + 2)              # O bf16, W bf16 r/w
    for k, by in (("momentum_norm", mom_bytes), ("param_update", upd_bytes)):
        if prof[k][1]:
            t = prof[k][0] / prof[k][1] * 1e-3
            hbm[k] = {"GBs": round(by / t / 1e9, 1), "frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
                      "bytes": by, "traffic": round(traffic[k]) if k in traffic else None}
    if prof["qk_rescale"][1]:
        # the clipped heads' rows of W_q and W_k, each read and written once
        # (bf16); 59 MB per step here, so the pass is launch-bound
        by = int((clipped == 1).sum()) * D * dm * 2 * 2 * 2
        t = prof["qk_rescale"][0] / prof["qk_rescale"][1] * 1e-3
        hbm["qk_rescale"] = {"GBs": round(by / t / 1e9, 1), "frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
                             "bytes": by, "traffic": round(traffic["qk_rescale"]) if "qk_rescale" in traffic else None}
    if prof["qk_rowmax"][1]:
        qk_flop = 2 * D * B * H * T * (T + 1) / 2
        t = prof["qk_rowmax"][0] / prof["qk_rowmax"][1] * 1e-3
        kernels["qk_rowmax"]["tflops"] = round(qk_flop / t / 1e12, 1)
        kernels["qk_rowmax"]["frac_mfma_peak"] = round(qk_flop / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)

    out = {
        "metric": "Muon steps/s + Newton–Schulz TFLOP/s (% bf16 MFMA peak), 1 MI355X",
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "MuonClip layer: hidden 7168, 64 heads x 128, batch 4 x seq 4096; "
                               "Muon step on W_q, W_k, W_v [8192x7168] and W_o [7168x8192]",
                   "ns_steps": wl.ns_steps, "tau": ex["tau"], "parallelism": "single GPU"},
        "ns_tflops": round(ns_tflops, 1),
        "ns_frac_mfma_peak": round(ns_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "ns_frac_measured_mfma_peak": round(ns_tflops / MFMA_BF16_MEASURED_TFLOPS, 4),
        "ns_ms_per_step": round(ns_ms_step, 3),
        "roofline": roofline,
        "hbm_passes": hbm,
        "kernels": kernels,
        "heads_clipped_per_step": n_clipped,
    }

    note("MuonClip layer step timed")
    out["companion"] = companion(mm, torch, dev, seed, n_mats * m * n)
    out["companion"]["attn_fwd"] = attention_companion(mm, torch, dev, seed, Q, K, B, T, H, D, prof["qk_rowmax"])
    del Q, K, Wqkv, Wo, Gqkv, Go, Mqkv, Mo, ws, groups
    torch.cuda.empty_cache()
    note("companion passes timed")
    out["layer_hidden2048"] = config_reading(mm, torch, dev, seed, 2, args.steps, args.warmup)
    note("hidden-2048 layer timed")
    out["single_matrix_256x128"] = small_matrix_reading(mm, torch, dev, seed)
    note("single 256x128 matrix timed")
    if not args.no_other_configs:
        k = max(2, min(3, args.steps))
        out["other_configs"] = {"dense_decoder_24_layers": config_reading(mm, torch, dev, seed, 3, k, 1)}
        note("24-layer decoder timed")
        out["other_configs"]["moe_64_experts"] = config_reading(mm, torch, dev, seed, 4, k, 1)
        note("64-expert MoE stack timed")
        out["dion_rank128"] = dion_reading(mm, torch, dev, seed)
        note("Dion step timed")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, m, n, n_mats, B, T, H, D)
    print(json.dumps(out), flush=True)


def blas_reference(torch, reps=10):
    """hipBLASLt (torch.matmul) on the three products of one Newton-Schulz
    iteration at the layer's shape (4 matrices, wide 7168 x 8192), computed
    in full (no symmetry) and without the a X / b A terms.  Operands are
    contiguous; the result is a reference point, not part of the method."""
    dev = torch.device("cuda:0")
    m, n, nb = 7168, 8192, 4
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    Bm = (torch.randn((nb, m, m), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    X = (torch.randn((nb, m, n), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    Xt = X.transpose(1, 2).contiguous()
    res = {"shapes": "4 x (7168x7168 @ 7168x8192, 7168x8192 @ 8192x7168, 7168x7168 @ 7168x7168)"}
    for name, f, flop in (("B_X", lambda: torch.matmul(Bm, X), 2.0 * nb * m * m * n),
                          ("X_Xt_full", lambda: torch.matmul(X, Xt), 2.0 * nb * m * m * n),
                          ("A_A_full", lambda: torch.matmul(Bm, Bm), 2.0 * nb * m * m * m)):
        f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"ms": round(ms, 3), "tflops": round(flop / ms / 1e9, 1)}
    res["ns_iteration_ms"] = round(sum(v["ms"] for k, v in res.items() if isinstance(v, dict)), 3)
    return res


def small_matrix_reading(mm, torch, dev, seed, steps=200, warmup=20):
    """The single fp32 256x128 matrix: 10 fresh N(0,1) gradients drawn on the
    device beforehand and cycled, W ~ N(0, 0.02^2), momentum from zero,
    Nesterov, 5 Newton-Schulz steps.  Latency-bound: one launch per step (the
    whole step in one workgroup); reported as microseconds per step, eagerly
    and replayed from a captured HIP graph."""
    from synthetic import generators as gen
    wl = gen.workload(1)
    gr = wl.groups[0]
    W = gen.bulk_normal_torch((gr.rows, gr.cols), wl.weight_std, seed + 500, dev, torch.float32)
    M = torch.zeros((gr.rows, gr.cols), dtype=torch.float32, device=dev)
    grads = [gen.bulk_normal_torch((gr.rows, gr.cols), 1.0, seed + 510 + k, dev, torch.float32)
             for k in range(10)]
    hp = mm.HParams(lr=wl.lr, momentum=wl.momentum, weight_decay=wl.weight_decay, nesterov=True,
                    ns_steps=wl.ns_steps, ns_coeffs=wl.ns_coeffs, ns_eps=wl.ns_eps, rms_target=wl.rms_target)
    ws = torch.empty(mm.workspace_size([(W, grads[0], M)]), dtype=torch.uint8, device=dev)
    for k in range(warmup):
        mm.muon_step([(W, grads[k % 10], M)], hp, workspace=ws)
    torch.cuda.synchronize()
    mm.profile_enable(True)
    t0 = time.perf_counter()
    for k in range(steps):
        mm.muon_step([(W, grads[k % 10], M)], hp, workspace=ws)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    prof = mm.profile_collect()
    mm.profile_enable(False)
    # one captured step on a side stream, replayed (the gradient buffer is fixed)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        mm.muon_step([(W, grads[0], M)], hp, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    el_graph = time.perf_counter() - t0
    return {"workload": "1 x 256x128 fp32, 5 Newton-Schulz steps", "steps": steps,
            "us_per_step": round(1e6 * el / steps, 2), "steps_per_s": round(steps / el, 1),
            "graph_us_per_step": round(1e6 * el_graph / steps, 2),
            "kernels_us_per_step": {k: round(1e3 * v[0] / steps, 2) for k, v in prof.items() if v[1]},
            "launches_per_step": sum(v[1] for v in prof.values()) / steps}


def dion_reading(mm, torch, dev, seed, batch=48, size=4096, rank=128, steps=3):
    """Dion's rank-r step next to the Muon step on the same group: 48 bf16
    4096 x 4096 matrices (the square class of the 24-layer decoder; 4096^2 is
    the pages' own example size for Dion's traffic), rank 128, fp32 momentum,
    N(0,1) gradients, Q column-normalised Gaussian.  Flops per matrix: the
    products B Q and B^T P (2 m n r each), P L^-T twice (2 m r^2 each) and the
    update's two rank-r products (4 m n r): 8 m n r + 4 m r^2."""
    from synthetic import generators as gen
    shape = (batch, size, size)
    W = gen.bulk_normal_torch(shape, 0.02, seed + 600, dev, torch.bfloat16)
    G = gen.bulk_normal_torch(shape, 1.0, seed + 601, dev, torch.bfloat16)
    M = gen.bulk_normal_torch(shape, 0.5, seed + 602, dev, torch.float32)
    Q = gen.bulk_normal_torch((batch, size, rank), 1.0, seed + 603, dev, torch.float32)
    Q /= Q.norm(dim=1, keepdim=True)
    ws = torch.empty(max(mm.load_library().dion_workspace_size(batch, size, size, rank), 256),
                     dtype=torch.uint8, device=dev)
    mm.dion_step(W, G, M, Q, lr=0.02, mu=0.95, workspace=ws)
    torch.cuda.synchronize()
    mm.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        mm.dion_step(W, G, M, Q, lr=0.02, mu=0.95, workspace=ws)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    prof = mm.profile_collect()
    mm.profile_enable(False)
    del ws
    torch.cuda.empty_cache()
    m = n = size
    flop = batch * (8.0 * m * n * rank + 4.0 * m * rank * rank)
    kflop = {"dion_bq": 2.0 * m * n * rank, "dion_btp": 2.0 * m * n * rank, "dion_update": 4.0 * m * n * rank,
             "dion_pl": 2.0 * m * rank * rank}
    kern = {}
    for k, v in prof.items():
        if not v[1]:
            continue
        kern[k] = {"ms_per_step": round(v[0] / steps, 4), "launches_per_step": v[1] / steps}
        if k in kflop:
            tf = batch * kflop[k] * (v[1] / steps) / (v[0] / steps * 1e-3) / 1e12
            kern[k]["tflops_fp32"] = round(tf, 1)
            kern[k]["frac_fp32_mfma_peak"] = round(tf / MFMA_FP32_PEAK_TFLOPS, 4)
    # the Muon step on the same group, for the comparison the pages make
    hp = mm.HParams(lr=0.02, momentum=0.95, weight_decay=0.0)
    mws = torch.empty(mm.workspace_size([(W, G, M)]), dtype=torch.uint8, device=dev)
    mm.muon_step([(W, G, M)], hp, workspace=mws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mm.muon_step([(W, G, M)], hp, workspace=mws)
    torch.cuda.synchronize()
    el_muon = time.perf_counter() - t0
    del W, G, M, Q, mws
    torch.cuda.empty_cache()
    return {"workload": f"{batch} x {size}x{size} bf16, rank {rank}", "steps": steps,
            "dion_ms_per_step": round(1e3 * el / steps, 3), "dion_steps_per_s": round(steps / el, 3),
            "dion_tflops_fp32": round(flop / (el / steps) / 1e12, 1),
            "muon_ms_per_step_same_group": round(1e3 * el_muon / steps, 3),
            "kernels": kern}


def config_reading(mm, torch, dev, seed, idx, steps, warmup):
    """The Muon step alone (no QK-Clip) on one of the other configurations,
    drawn on the GPU with its recipe (bf16 params and grads, fp32 momentum;
    grads N(0,1), low-rank-plus-noise, or low-rank-plus-noise with Zipf(1.1)
    expert magnitudes).  A second reading of the same metric beside the
    headline MuonClip layer, whose step is the only one that covers every
    stage of the path."""
    from synthetic import generators as gen
    wl = gen.workload(idx)
    groups = []
    for gi, gr in enumerate(wl.groups):
        W = gen.bulk_normal_torch((gr.batch, gr.rows, gr.cols), 0.02, seed + 100 + gi, dev, torch.bfloat16)
        if wl.grad_kind == "normal":
            G = gen.bulk_normal_torch((gr.batch, gr.rows, gr.cols), 1.0, seed + 200 + gi, dev, torch.bfloat16)
        else:
            mags = gen.zipf_magnitudes(gen.rng(seed + 7), gr.batch) if wl.grad_kind == "lowrank_zipf" \
                else [1.0] * gr.batch
            G = torch.stack([gen.lowrank_torch(gr.rows, gr.cols, seed + 200 + 1000 * gi + b, dev,
                                               magnitude=float(mags[b])) for b in range(gr.batch)])
        M = gen.bulk_normal_torch((gr.batch, gr.rows, gr.cols), 0.5, seed + 300 + gi, dev, torch.float32)
        groups.append((W, G, M))
    hp = mm.HParams(lr=wl.lr, momentum=wl.momentum, weight_decay=wl.weight_decay, nesterov=True,
                    ns_steps=wl.ns_steps, ns_coeffs=wl.ns_coeffs, ns_eps=wl.ns_eps, rms_target=wl.rms_target)
    ws = torch.empty(mm.workspace_size(groups), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        mm.muon_step(groups, hp, workspace=ws)
    torch.cuda.synchronize()
    mm.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        mm.muon_step(groups, hp, workspace=ws)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    prof = mm.profile_collect()
    mm.profile_enable(False)
    flop = 0.0
    for gr in wl.groups:
        m, n = min(gr.rows, gr.cols), max(gr.rows, gr.cols)
        flop += gr.batch * wl.ns_steps * sum(ns_flops(m, n).values())
    ns_ms = sum(prof[k][0] for k in ("ns_syrk_xxt", "ns_syrk_poly", "ns_gemm_bx",
                                     "ns_syrk_xxt_slices", "ns_syrk_poly_slices") if k in prof) / steps
    res = {"workload": wl.name + ": " + ", ".join(f"{g.batch} x {g.rows}x{g.cols}" for g in wl.groups),
           "steps": steps, "steps_per_s": round(steps / el, 3), "ms_per_step": round(1e3 * el / steps, 3),
           "ns_tflops": round(flop / (ns_ms * 1e-3) / 1e12, 1),
           "ns_frac_mfma_peak": round(flop / (ns_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "kernels_ms_per_step": {k: round(v[0] / steps, 4) for k, v in prof.items() if v[1]}}
    del groups, ws
    torch.cuda.empty_cache()
    return res


def attention_companion(mm, torch, dev, seed, Q, K, B, T, H, D, rowmax_prof, reps=5):
    """The causal attention forward on the layer's Q, K and a synthetic V,
    which produces the same S_max as the separate rowmax pass.  Algorithmic
    work: two products over the causal pairs, 4 d B H T (T + 1) / 2 flops."""
    from synthetic import generators as gen
    V = gen.bulk_normal_torch((B, T, H, D), 1.0, seed + 40, dev, torch.bfloat16)
    out = torch.empty_like(Q)
    s_max = torch.empty(H, dtype=torch.float32, device=dev)
    ws = torch.empty(max(mm.load_library().attn_fwd_workspace_size(B, T, H), 256), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    mm.attn_fwd(Q, K, V, scale, True, out=out, s_max=s_max, workspace=ws)
    torch.cuda.synchronize()
    mm.profile_enable(True)
    for _ in range(reps):
        mm.attn_fwd(Q, K, V, scale, True, out=out, s_max=s_max, workspace=ws)
    prof = mm.profile_collect()
    mm.profile_enable(False)
    ms, cnt = prof["attn_fwd"]
    t = ms / cnt * 1e-3
    flop = 4.0 * D * B * H * T * (T + 1) / 2
    res = {"avg_us": round(1e6 * t, 1), "tflops": round(flop / t / 1e12, 1),
           "frac_mfma_peak": round(flop / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    if rowmax_prof[1]:
        res["separate_rowmax_pass_us"] = round(1e3 * rowmax_prof[0] / rowmax_prof[1], 1)
    del V, out
    return res


def companion(mm, torch, dev, seed, n_elem, reps=5):
    """The parts of a full MuonClip step that sit beside the timed Muon path,
    timed on their own after it: AdamW over as many parameters as the layer's
    four matrices hold (bf16 params and grads, fp32 moments: 22 bytes per
    element) plus two norm weights, and the MLA QK-Clip rescale at a
    latent-attention shape (64 heads, content 128 and rotary 64 rows per head,
    query latent 1536, key/value latent 512, every head clipped)."""
    from synthetic import generators as gen
    hd, H, d_c, d_r, q_in, kv_in = 7168, 64, 128, 64, 1536, 512
    P = [gen.bulk_normal_torch((n_elem,), 0.02, seed + 20, dev, torch.bfloat16),
         torch.ones(hd, dtype=torch.bfloat16, device=dev), torch.ones(hd, dtype=torch.bfloat16, device=dev)]
    G = [gen.bulk_normal_torch((t.numel(),), 1e-3, seed + 21 + i, dev, torch.bfloat16) for i, t in enumerate(P)]
    M = [torch.zeros(t.numel(), dtype=torch.float32, device=dev) for t in P]
    V = [torch.zeros(t.numel(), dtype=torch.float32, device=dev) for t in P]
    Wqc = gen.bulk_normal_torch((H * d_c, q_in), 0.02, seed + 30, dev, torch.bfloat16)
    Wkc = gen.bulk_normal_torch((H * d_c, kv_in), 0.02, seed + 31, dev, torch.bfloat16)
    Wqr = gen.bulk_normal_torch((H * d_r, q_in), 0.02, seed + 32, dev, torch.bfloat16)
    s_hi = torch.full((H,), 1.0e4, dtype=torch.float32, device=dev)
    mm.adamw_step(P, G, M, V, lr=3e-4, step=1)
    mm.qkclip_rescale_mla(Wqc, Wkc, Wqr, s_hi, d_c, d_r)
    torch.cuda.synchronize()
    mm.profile_enable(True)
    for t in range(reps):
        mm.adamw_step(P, G, M, V, lr=3e-4, step=t + 2)
        mm.qkclip_rescale_mla(Wqc, Wkc, Wqr, s_hi, d_c, d_r)
    prof = mm.profile_collect()
    mm.profile_enable(False)
    res = {}
    n_all = sum(t.numel() for t in P)
    ms, cnt = prof["adamw"]
    if cnt:
        by = 22 * n_all
        t = ms / cnt * 1e-3
        res["adamw"] = {"params": n_all, "avg_us": round(1e6 * t, 1), "bytes": by,
                        "GBs": round(by / t / 1e9, 1), "frac_hbm_peak": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
    ms, cnt = prof["qk_rescale"]
    if cnt:
        by = 2 * 2 * H * (d_c * q_in + d_c * kv_in + d_r * q_in)   # bf16 read + write
        t = ms / cnt * 1e-3
        res["qkclip_rescale_mla"] = {"avg_us": round(1e6 * t, 2), "bytes": by,
                                     "GBs": round(by / t / 1e9, 1)}
    del P, G, M, V, Wqc, Wkc, Wqr
    return res


def cpu_baseline(wl, m, n, n_mats, B, T, H, D):
    """Time the fp64 oracle on a bounded sample and extrapolate to one step:
    one Newton-Schulz iteration, the momentum and update of one 7168 x 8192
    matrix, and the causal logit maximum of one (batch row, head) pair."""
    import numpy as np

    from oracle import muon_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    g = np.random.default_rng(1)
    X = g.standard_normal((m, n))
    X /= np.linalg.norm(X)
    t0 = time.perf_counter()
    O.newton_schulz_iterate(X, 1, *wl.ns_coeffs)
    t_iter = time.perf_counter() - t0
    W = g.standard_normal((m, n)) * 0.02
    M = g.standard_normal((m, n)) * 0.5
    G = g.standard_normal((m, n))
    t0 = time.perf_counter()
    Mn = O.momentum_update(M, G, wl.momentum)
    U = O.nesterov_lookahead(Mn, G, wl.momentum, True)
    O.frobenius_normalize(U, wl.ns_eps)
    O.param_update(W, U, wl.lr, wl.weight_decay, 18.1)
    t_elem = time.perf_counter() - t0
    Qs = g.standard_normal((1, T, 1, D))
    Ks = g.standard_normal((1, T, 1, D))
    t0 = time.perf_counter()
    O.smax_per_head(Qs, Ks, 1 / math.sqrt(D), True)
    t_pair = time.perf_counter() - t0
    step_s = n_mats * (wl.ns_steps * t_iter + t_elem) + B * H * t_pair
    return {"value": round(1.0 / step_s, 6), "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 NumPy oracle: 1 Newton-Schulz iteration ({t_iter:.2f} s) and the "
                       f"momentum/normalise/update pass ({t_elem:.2f} s) of one 7168x8192 matrix, "
                       f"S_max of one (batch row, head) pair ({t_pair:.2f} s); extrapolated to "
                       f"{n_mats} matrices x {wl.ns_steps} iterations + {B * H} pairs"),
            "seconds_per_step": round(step_s, 2)}


if __name__ == "__main__":
    main()
