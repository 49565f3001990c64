"""Benchmark: the Muon step of a 24-layer dense decoder on one MI355X.

The headline step is the whole Muon path on the decoder's Muon group (hidden
4096, 32 query / 8 KV heads of 128, FFN 14336; per layer W_q, W_o 4096x4096,
W_k, W_v 1024x4096, up and gate 14336x4096, down 4096x14336; 168 matrices,
bf16 params and grads, fp32 momentum): the momentum + Nesterov + Frobenius
pass, 5 quintic Newton-Schulz iterations as bf16 MFMA GEMMs batched by shape
class, and the scaled, decayed parameter write.  It is the largest workload
that fits one GPU.  The MuonClip attention layer (per-head causal max-logit
statistic on the forward's Q and K, Muon step on W_q, W_k, W_v [8192x7168] and
W_o [7168x8192], per-head rescale at tau = 100), the hidden-2048 layer, the
64-expert MoE stack and the single 256x128 fp32 matrix are reported beside it.

Inputs are seeded and synthetic and resident in HBM before timing.  Per-kernel
times come from HIP events the library records around each launch on the
benchmark stream.  The CPU baseline times the fp64 oracle on a bounded sample
(one matrix per shape class) and extrapolates to one step.

Prints one JSON line on stdout; progress lines go to stderr.
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
HBM_PEAK_GBS = 8000.0
MFMA_FP32_PEAK_TFLOPS = 157.3    # dense fp32 MFMA, the spec figure
NS_KINDS = ("ns_syrk_xxt", "ns_syrk_poly", "ns_gemm_bx")
SLICE_KINDS = ("ns_syrk_xxt_slices", "ns_syrk_poly_slices")
THIN_KINDS = ("ns_thin_gram", "ns_thin_poly", "ns_thin_bx")
HEADLINE_TRAFFIC = os.path.join("profiles", "decoder24_step_hbm_traffic.txt")
LAYER_TRAFFIC = os.path.join("profiles", "muonclip_layer_step_hbm_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the decoder step alone (for profiler runs)")
    ap.add_argument("--layer-only", action="store_true",
                    help="time the MuonClip layer step alone (for profiler runs)")
    ap.add_argument("--attention-only", action="store_true",
                    help="time the attention forward with its S_max export alone, at the MuonClip "
                         "layer's shape (for profiler runs)")
    ap.add_argument("--seed", type=int, default=5000)
    ap.add_argument("--blas-reference", action="store_true",
                    help="time torch.matmul (hipBLASLt) on the full, unsymmetric Newton-Schulz "
                         "products of the MuonClip layer's shape, for comparison, and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (to scale HBM counters)")
    ap.add_argument("--summarize-profile", nargs="+", metavar="CSV",
                    help="print a per-kernel summary of rocprofv3 kernel-trace or counter CSV "
                         "files and exit (no GPU use)")
    ap.add_argument("--summarize-clock", nargs="+", metavar="CSV",
                    help="print each kernel's shader clock and MFMA busy share from rocprofv3 counter "
                         "CSVs of GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES and exit (no GPU use)")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs, "
                         "scaled by the same counters of the 1 GiB copy (--copy-calibration); "
                         "prints a table and a TRAFFIC_JSON line, then exits (no GPU use)")
    return ap.parse_args()


def note(msg):
    """A progress line on stderr (the JSON result alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def ns_flops(m, n):
    """Algorithmic flops of one Newton-Schulz iteration on a wide m x n matrix
    with the symmetric products counted once: X X^T (upper triangle incl.
    diagonal: m(m+1)/2 dots of length n), A A^T (m(m+1)/2 dots of length m),
    B X (m n dots of length m)."""
    return {"ns_syrk_xxt": m * (m + 1) * n, "ns_syrk_poly": m * m * (m + 1), "ns_gemm_bx": 2 * m * m * n}


def ns_flops_dense(m, n):
    """The pages' count for one iteration, 2 (2 n m^2 + m^3) ("Muon and
    MuonClip", Newton-Schulz cost paragraph): every product in full."""
    return 2 * (2 * n * m * m + m ** 3)


def measured_traffic(path):
    """Per-launch HBM bytes from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, keyed by kernel; an entry is used only while the hash of its
    kernel source still matches the source the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, path)
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


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_clock:
        summarize_clock(args.summarize_clock)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 "
                                   "(the step would shard by whole matrices across GPUs; no multi-GPU path "
                                   "is implemented)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    if args.copy_calibration:
        print(json.dumps(copy_calibration(torch)))
        return
    if args.blas_reference:
        print(json.dumps(blas_reference(torch)), flush=True)
        return

    import matrix_orthogonalizing_optimizer_muon_amd as mm
    dev = torch.device("cuda:0")
    seed = args.seed

    if args.layer_only:
        res = muonclip_layer_reading(mm, torch, dev, seed, args.steps, args.warmup)
        print(json.dumps(res), flush=True)
        return
    if args.attention_only:
        from synthetic import generators as gen
        B, T, H, D = 4, 4096, 64, 128
        Q = gen.bulk_normal_torch((B, T, H, D), 1.0, seed + 41, dev, torch.bfloat16)
        K = gen.bulk_normal_torch((B, T, H, D), 1.0, seed + 42, dev, torch.bfloat16)
        res = attention_companion(mm, torch, dev, seed, Q, K, B, T, H, D, (0.0, 0), reps=args.steps)
        print(json.dumps({"workload": f"attention forward with S_max, B {B} x T {T} x H {H} x d {D}, causal",
                          **res}), flush=True)
        return

    # ---------------- headline: the 24-layer decoder's Muon group
    head = muon_config_run(mm, torch, dev, seed, 3, args.steps, args.warmup, roofline=True)
    note("24-layer decoder step timed")
    out_sigma = None if args.headline_only else sigma_band(mm, torch, dev, seed)
    # the matrix-core probe runs after the headline, on a GPU already at its working clock
    peak = None if args.headline_only else mfma_peak(mm, torch, dev)
    if peak:
        note(f"register-only MFMA loop: {peak['tflops']} TFLOP/s on random operands, "
             f"{peak['smooth_operands_tflops']} on smooth ones")
    out = {
        "metric": "Muon steps/s + Newton–Schulz TFLOP/s (% bf16 MFMA peak), 1 MI355X",
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "ns_steps": 5, "matrices": head["matrices"],
                   "parallelism": "single GPU"},
    }
    for k in ("median_ms_per_step", "ns_tflops", "ns_frac_mfma_peak", "ns_ms_per_step",
              "ns_tflops_dense_equivalent", "roofline", "hbm_passes", "kernels"):
        out[k] = head[k]
    if peak:
        out["mfma_measured_peak"] = peak
        out["ns_frac_measured_mfma_peak"] = round(head["ns_tflops"] / peak["tflops"], 4)
        out["roofline"]["measured_peak"] = peak["tflops"]
        out["roofline"]["frac_of_measured_peak"] = round(out["roofline"]["achieved"] / peak["tflops"], 4)
    if out_sigma:
        out["ns_sigma_band"] = out_sigma
    torch.cuda.empty_cache()
    hbm = None if args.headline_only else hbm_stream_rates(mm, torch, dev)
    if hbm:
        out["hbm_stream_probe"] = hbm
        attach_hbm_probe(out["hbm_passes"], hbm)
        note(f"HBM stream probe: {hbm['mix_6r_8w_GBs']} GB/s for the momentum pass's mix, "
             f"{hbm['mix_4r_2w_GBs']} for the update's, {hbm['copy_GBs']} for a copy")

    if not args.headline_only:
        out["muonclip_layer"] = muonclip_layer_reading(mm, torch, dev, seed, args.steps, args.warmup,
                                                       companions=True)
        if hbm:
            attach_hbm_probe(out["muonclip_layer"]["hbm_passes"], hbm)
        note("MuonClip layer step timed")
        out["layer_hidden2048"] = muon_config_run(mm, torch, dev, seed, 2, args.steps, args.warmup)
        note("hidden-2048 layer timed")
        out["moe_64_experts"] = muon_config_run(mm, torch, dev, seed, 4, args.steps, args.warmup)
        note("64-expert MoE stack timed")
        out["single_matrix_256x128"] = small_matrix_reading(mm, torch, dev, seed)
        note("single 256x128 matrix timed")
        out["dion_rank128"] = dion_reading(mm, torch, dev, seed)
        note("Dion step timed")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decoder(seed)
        note("CPU baseline timed")
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# readings
# ---------------------------------------------------------------------------

def mfma_peak(mm, torch, dev, iters=8000):
    """The register-only MFMA loop on every CU (two 256-thread blocks per CU,
    one wave per SIMD each, eight accumulators per wave), timed with events:
    the sustained bf16 matrix-core rate at the clock the chip holds under that
    load.  The matrix cores draw more power, and the chip holds a lower clock,
    on random operands than on smooth ones; the random-operand rate is the one
    the Newton-Schulz products are compared with (their operands are
    random-like).  About 80 ms of warm-up, then the best of 3 runs per kind."""
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * ncu
    sink = torch.empty(blocks, dtype=torch.float32, device=dev)
    for _ in range(8):
        mm.mfma_probe(blocks, iters, sink, mm.PROBE_RANDOM)
    torch.cuda.synchronize()
    best = {}
    for kind in (mm.PROBE_RANDOM, mm.PROBE_SMOOTH):
        best[kind] = 0.0
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            flop = mm.mfma_probe(blocks, iters, sink, kind)
            e1.record()
            torch.cuda.synchronize()
            best[kind] = max(best[kind], flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    r = best[mm.PROBE_RANDOM]
    return {"tflops": round(r, 1), "frac_of_spec": round(r / MFMA_BF16_PEAK_TFLOPS, 4),
            "smooth_operands_tflops": round(best[mm.PROBE_SMOOTH], 1),
            "probe": f"{blocks} blocks x 4 waves x 32 x {iters} v_mfma_f32_32x32x16_bf16 on random bf16 "
                     "register operands (smooth operands beside it), best of 3 after ~80 ms of warm-up"}


def hbm_stream_rates(mm, torch, dev, gib=3):
    """The HBM stream probe (muon_hbm_probe) on `gib` GiB streams for the
    read/write mixes of the two passes and a plain copy: 6 B read and 8 B
    written per element (the momentum pass with its transposed X0 copy),
    4 B read and 2 B written (the update pass), 1:1.  Best of 3 timed
    launches after 3 warm-up launches per mix and launch shape (1 or 4 units
    per thread), HIP events on the current stream."""
    n = gib << 30
    src = torch.empty(n // 4, dtype=torch.int32, device=dev)
    src.random_()
    dst = torch.empty(n // 4, dtype=torch.int32, device=dev)
    res = {}
    for key, r, w in (("mix_6r_8w_GBs", 3, 4), ("mix_4r_2w_GBs", 2, 1), ("copy_GBs", 1, 1)):
        best = 0.0
        for unroll in (1, 4):
            for _ in range(3):
                mm.hbm_probe(src, dst, r, w, unroll)
            for _ in range(3):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                moved = mm.hbm_probe(src, dst, r, w, unroll)
                e1.record()
                torch.cuda.synchronize()
                best = max(best, moved / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        res[key] = round(best, 1)
    del src, dst
    torch.cuda.empty_cache()
    res["probe"] = (f"nontemporal 16-byte loads and stores, 1 KB per wave instruction, {gib} GiB streams, "
                    "1 or 4 units per thread, best of 3 after 3 warm-up launches per mix and shape")
    return res


def attach_hbm_probe(passes, hbm):
    """Each HBM pass's moved bytes against the probe's rate for its mix."""
    for k, key in (("momentum_norm", "mix_6r_8w_GBs"), ("param_update", "mix_4r_2w_GBs")):
        if k in passes and hbm.get(key):
            passes[k]["frac_of_stream_probe"] = round(passes[k]["GBs_moved"] / hbm[key], 4)


def make_config_groups(mm, torch, dev, seed, idx):
    """The groups of one workload drawn on the GPU with its recipe (bf16
    params and grads, fp32 momentum; grads N(0,1), low-rank-plus-noise, or
    low-rank-plus-noise with Zipf(1.1) expert magnitudes)."""
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
    return wl, groups, hp


def timed_steps(mm, torch, step, steps, warmup):
    """W untimed steps, then exactly K timed steps between two device
    synchronisations, with an event per step for the median; the library's
    per-kernel events are recorded meanwhile."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    mm.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for k in range(steps):
        step()
        ev[k + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = mm.profile_collect()
    mm.profile_enable(False)
    per = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(steps))
    median = per[len(per) // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    return elapsed, median, prof


def ns_summary(wl, prof, steps):
    """Newton-Schulz flops and time per step over the tiled and thin products."""
    flop = dense = 0.0
    per_kind = {k: 0.0 for k in NS_KINDS}
    for gr in wl.groups:
        m, n = min(gr.rows, gr.cols), max(gr.rows, gr.cols)
        f = ns_flops(m, n)
        for k in NS_KINDS:
            per_kind[k] += gr.batch * wl.ns_steps * f[k]
        flop += gr.batch * wl.ns_steps * sum(f.values())
        dense += gr.batch * wl.ns_steps * ns_flops_dense(m, n)
    ns_ms = sum(prof[k][0] for k in NS_KINDS + SLICE_KINDS + THIN_KINDS if k in prof) / steps
    return flop, dense, per_kind, ns_ms


def muon_config_run(mm, torch, dev, seed, idx, steps, warmup, roofline=False):
    """The Muon step alone on one workload, all its groups in one call."""
    wl, groups, hp = make_config_groups(mm, torch, dev, seed, idx)
    ws = torch.empty(mm.workspace_size(groups), dtype=torch.uint8, device=dev)
    elapsed, median, prof = timed_steps(mm, torch, lambda: mm.muon_step(groups, hp, workspace=ws), steps, warmup)
    flop, dense, per_kind, ns_ms = ns_summary(wl, prof, steps)
    nmat = sum(g.batch for g in wl.groups)
    res = {"workload": wl.name + ": " + ", ".join(f"{g.batch} x {g.rows}x{g.cols}" for g in wl.groups),
           "matrices": nmat, "steps": steps, "warmup": warmup,
           "steps_per_s": round(steps / elapsed, 3), "ms_per_step": round(1e3 * elapsed / steps, 3),
           "median_ms_per_step": round(median, 3),
           "ns_ms_per_step": round(ns_ms, 3),
           "ns_tflops": round(flop / (ns_ms * 1e-3) / 1e12, 1),
           "ns_frac_mfma_peak": round(flop / (ns_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "ns_tflops_dense_equivalent": round(dense / (ns_ms * 1e-3) / 1e12, 1),
           "kernels": {k: {"ms_per_step": round(v[0] / steps, 4), "launches_per_step": v[1] / steps,
                           "avg_us": round(1e3 * v[0] / v[1], 2)} for k, v in prof.items() if v[1]}}
    elem = sum(g.batch * g.rows * g.cols for g in wl.groups)
    res["hbm_passes"] = hbm_passes(prof, elem, HEADLINE_TRAFFIC if idx == 3 else None)
    if roofline:
        res["roofline"] = product_roofline(prof, per_kind, steps, HEADLINE_TRAFFIC)
    del groups, ws
    torch.cuda.empty_cache()
    return res


def sigma_band(mm, torch, dev, seed, band=(0.68, 1.2)):
    """Singular values of the Newton-Schulz output for one matrix of each of
    the 24-layer decoder's shape classes (N(0,1) gradients, 5 quintic steps),
    from the eigenvalues of O O^T (wide view) in fp64 on the GPU: minimum,
    median, maximum and the share inside the band the tuned quintic leaves
    them in ("Muon and MuonClip", Newton-Schulz interactive demo)."""
    from synthetic import generators as gen
    out = {}
    for i, (r, c) in enumerate(((4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336))):
        G = gen.bulk_normal_torch((r, c), 1.0, seed + 900 + i, dev, torch.float32)
        O = mm.ns_orthogonalize(G).double()
        W = O if r <= c else O.t()
        sv = torch.sqrt(torch.clamp(torch.linalg.eigvalsh(W @ W.t()), min=0.0))
        inside = ((sv >= band[0]) & (sv <= band[1])).double().mean()
        out[f"{r}x{c}"] = {"min": round(float(sv.min()), 4), "median": round(float(sv.median()), 4),
                           "max": round(float(sv.max()), 4), "frac_in_band": round(float(inside), 4)}
        del G, O, W, sv
    torch.cuda.empty_cache()
    return {"band": list(band), "classes": out}


def product_roofline(prof, per_kind, steps, traffic_path):
    """The dominant Newton-Schulz product: its algorithmic flops per launch
    (flops per step over launches per step) over its average launch time."""
    ms = {k: prof[k][0] + prof.get(k + "_slices", (0.0, 0))[0] for k in NS_KINDS if k in prof}
    dom = max(ms, key=ms.get)
    launches = prof[dom][1] + prof.get(dom + "_slices", (0.0, 0))[1]
    avg_s = ms[dom] / launches * 1e-3
    flop_launch = per_kind[dom] * steps / launches
    achieved = flop_launch / avg_s / 1e12
    traffic = measured_traffic(traffic_path)
    return {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": round(traffic[dom]) if dom in traffic else None,
            "flop_per_launch": flop_launch, "avg_launch_us": round(avg_s * 1e6, 1), "launches": launches}


def hbm_passes(prof, elem, traffic_path):
    """Algorithmic bytes per launch over the event time of the HBM passes:
    momentum + lookahead + Frobenius partials, 12 B per element for bf16
    gradients (G 2, M read 4 and written 4, X0 2); the scaled, decayed write,
    6 B per element (O 2, W read 2 and written 2).  The momentum pass also
    writes X0 transposed (2 B more per element), which the Newton-Schulz
    products read; that is reported as bytes_moved but not counted as work."""
    traffic = measured_traffic(traffic_path) if traffic_path else {}
    out = {}
    for k, per, moved in (("momentum_norm", 12, 14), ("param_update", 6, 6)):
        if k in prof and prof[k][1]:
            launches = prof[k][1]
            t = prof[k][0] / launches * 1e-3
            by = per * elem
            out[k] = {"GBs": round(by / t / 1e9, 1), "frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
                      "bytes": by, "bytes_per_element": per, "bytes_moved": moved * elem,
                      "GBs_moved": round(moved * elem / t / 1e9, 1), "avg_us": round(t * 1e6, 1),
                      "traffic": round(traffic[k]) if k in traffic else None}
    return out


def muonclip_layer_reading(mm, torch, dev, seed, steps, warmup, companions=False):
    """The MuonClip attention layer (hidden 7168, 64 heads x 128, batch 4 x seq
    4096): S_max on the forward's Q and K, the Muon step on W_q, W_k, W_v
    [8192x7168] and W_o [7168x8192], then the per-head W_q / W_k rescale."""
    import numpy as np
    from synthetic import generators as gen
    wl = gen.workload(5)
    ex = wl.extra
    B, T, H, D, dm = ex["batch"], ex["seq"], ex["heads"], ex["d_head"], ex["d_model"]
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

    def step():
        mm.qkclip_rowmax(Q, K, 1.0 / math.sqrt(D), True, out=s_max, workspace=rm_ws)
        mm.muon_step(groups, hp, workspace=ws)
        mm.qkclip_rescale(Wqkv[0], Wqkv[1], s_max, D, ex["tau"], ex["alpha"], clipped=clipped)

    elapsed, median, prof = timed_steps(mm, torch, step, steps, warmup)
    flop, dense, per_kind, ns_ms = ns_summary(wl, prof, steps)
    res = {"workload": "MuonClip layer: hidden 7168, 64 heads x 128, batch 4 x seq 4096; S_max, Muon step on "
                       "W_q, W_k, W_v [8192x7168] and W_o [7168x8192], per-head rescale at tau 100",
           "steps": steps, "warmup": warmup, "steps_per_s": round(steps / elapsed, 3),
           "ms_per_step": round(1e3 * elapsed / steps, 3), "median_ms_per_step": round(median, 3),
           "ns_ms_per_step": round(ns_ms, 3), "ns_tflops": round(flop / (ns_ms * 1e-3) / 1e12, 1),
           "ns_frac_mfma_peak": round(flop / (ns_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "ns_tflops_dense_equivalent": round(dense / (ns_ms * 1e-3) / 1e12, 1),
           "heads_clipped_per_step": int((clipped == 1).sum())}
    # the step's telemetry (read after timing): the per-head statistic and the clip factors
    sm = s_max.float().cpu().numpy()
    fl = clipped.cpu().numpy()
    clip_heads = [int(h) for h in range(H) if fl[h] == 1]
    res["telemetry"] = {"s_max_min": round(float(sm.min()), 3), "s_max_median": round(float(np.median(sm)), 3),
                        "s_max_max": round(float(sm.max()), 3), "tau": ex["tau"], "clipped_heads": clip_heads,
                        "gamma_min": round(float(ex["tau"] / sm[clip_heads].max()), 5) if clip_heads else None}
    res["roofline"] = product_roofline(prof, per_kind, steps, LAYER_TRAFFIC)
    res["hbm_passes"] = hbm_passes(prof, 4 * 7168 * 8192, LAYER_TRAFFIC)
    kern = {k: {"ms_per_step": round(v[0] / steps, 4), "launches_per_step": v[1] / steps,
                "avg_us": round(1e3 * v[0] / v[1], 2)} for k, v in prof.items() if v[1]}
    if prof["qk_rowmax"][1]:
        # the statistic is a max over every causal pair: 2 d B H T (T + 1) / 2 flops
        qk_flop = 2 * D * B * H * T * (T + 1) / 2
        t = prof["qk_rowmax"][0] / prof["qk_rowmax"][1] * 1e-3
        kern["qk_rowmax"]["tflops"] = round(qk_flop / t / 1e12, 1)
        kern["qk_rowmax"]["frac_mfma_peak"] = round(qk_flop / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        kern["qk_rowmax"]["bytes_read"] = 2 * B * T * H * D * 2
    if prof["qk_reduce"][1]:
        # per-head reduction of the row-max pass's partial maxima: B H ceil(T / q)
        # fp32 partials read (q = 512 queries per block for d = 128, else 256),
        # H fp32 written; launch-bound at this size
        q = 512 if D == 128 else 256
        by = 4 * (B * H * ((T + q - 1) // q) + H)
        t = prof["qk_reduce"][0] / prof["qk_reduce"][1] * 1e-3
        kern["qk_reduce"]["bytes"] = by
        kern["qk_reduce"]["GBs"] = round(by / t / 1e9, 2)
    if prof["qk_rescale"][1]:
        # the clipped heads' rows of W_q and W_k, each read and written once (bf16)
        by = res["heads_clipped_per_step"] * D * dm * 2 * 2 * 2
        t = prof["qk_rescale"][0] / prof["qk_rescale"][1] * 1e-3
        kern["qk_rescale"]["bytes"] = by
        kern["qk_rescale"]["GBs"] = round(by / t / 1e9, 1)
    res["kernels"] = kern
    if companions:
        res["companion"] = companion(mm, torch, dev, seed, 4 * 7168 * 8192)
        res["companion"]["attn_fwd"] = attention_companion(mm, torch, dev, seed, Q, K, B, T, H, D,
                                                           prof["qk_rowmax"])
    del Q, K, Wqkv, Wo, Gqkv, Go, Mqkv, Mo, ws, groups
    torch.cuda.empty_cache()
    return res


def copy_calibration(torch):
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
    return {"copy_calibration_bytes": src.numel(), "copies": 3,
            "copy_GBs_read_plus_write": round(2 * src.numel() / ms / 1e6, 1)}


def blas_reference(torch, reps=10):
    """hipBLASLt (torch.matmul) on the three products of one Newton-Schulz
    iteration, computed in full (no symmetry) and without the a X / b A terms,
    at the MuonClip layer's shape (4 matrices, wide 7168 x 8192) and at the
    24-layer decoder's largest shape class (72 matrices, wide 4096 x 14336).
    Operands are contiguous; the result is a reference point, not part of the
    method."""
    dev = torch.device("cuda:0")
    out = {}
    for key, m, n, nb in (("muonclip_layer", 7168, 8192, 4), ("decoder_4096x14336", 4096, 14336, 72)):
        g = torch.Generator(device=dev)
        g.manual_seed(1)
        Bm = (torch.randn((nb, m, m), generator=g, device=dev) * 0.01).to(torch.bfloat16)
        X = (torch.randn((nb, m, n), generator=g, device=dev) * 0.01).to(torch.bfloat16)
        Xt = X.transpose(1, 2).contiguous()
        res = {"shapes": f"{nb} x ({m}x{m} @ {m}x{n}, {m}x{n} @ {n}x{m}, {m}x{m} @ {m}x{m})"}
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
        out[key] = res
        del Bm, X, Xt
        torch.cuda.empty_cache()
    return out


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


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores
# ---------------------------------------------------------------------------

def blas_info():
    """Threads and vendor of the BLAS NumPy calls (threadpoolctl), or
    numpy.show_config()'s build entry when threadpoolctl has nothing."""
    threads, vendor = os.cpu_count() or 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            threads = max(i.get("num_threads", 1) for i in blas)
            vendor = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in blas)
    except Exception:
        pass
    if vendor == "unknown":
        try:
            import numpy as np
            cfg = np.show_config(mode="dicts")
            vendor = str(cfg.get("Build Dependencies", {}).get("blas", {}).get("name", "unknown"))
        except Exception:
            pass
    return threads, vendor


def cpu_baseline_decoder(seed, iters=2):
    """Time the fp64 oracle on a bounded sample of the headline workload and
    extrapolate to one step: per shape class of the 24-layer decoder, `iters`
    Newton-Schulz iterations (timed together, averaged) and the momentum /
    lookahead / normalisation / update pass of one matrix; a step is each
    class's matrix count times (5 iterations + that pass).  Inputs are N(0, 1) draws of the class's
    shape (the oracle's time does not depend on the values)."""
    import numpy as np

    from oracle import muon_oracle as O
    from synthetic import generators as gen
    wl = gen.workload(3)
    threads, vendor = blas_info()
    g = np.random.default_rng(seed)
    step_s, parts = 0.0, []
    t_all = time.perf_counter()
    for gr in wl.groups:
        W = g.standard_normal((gr.rows, gr.cols)) * 0.02
        M = g.standard_normal((gr.rows, gr.cols)) * 0.5
        G = g.standard_normal((gr.rows, gr.cols))
        t0 = time.perf_counter()
        Mn = O.momentum_update(M, G, wl.momentum)
        U = O.nesterov_lookahead(Mn, G, wl.momentum, True)
        X, _ = O.to_wide(U)
        X = O.frobenius_normalize(X, wl.ns_eps)
        t_elem = time.perf_counter() - t0
        t0 = time.perf_counter()
        X = O.newton_schulz_iterate(X, iters, *wl.ns_coeffs)
        t_iter = (time.perf_counter() - t0) / iters
        t0 = time.perf_counter()
        O.param_update(W, X.T if gr.rows > gr.cols else X, wl.lr, wl.weight_decay,
                       O.update_scale(gr.rows, gr.cols))
        t_elem += time.perf_counter() - t0
        step_s += gr.batch * (wl.ns_steps * t_iter + t_elem)
        parts.append(f"{gr.rows}x{gr.cols}: {t_iter:.2f} s per iteration (mean of {iters}) + {t_elem:.2f} s")
    sample_s = time.perf_counter() - t_all
    return {"value": round(1.0 / step_s, 6), "unit": "steps/s", "cores": threads, "kind": "oracle",
            "blas": vendor,
            "sample": (f"fp64 NumPy oracle, one matrix per shape class of the 24-layer decoder ("
                       + "; ".join(parts) + f"), {sample_s:.1f} s in all; extrapolated to "
                       f"{sum(g.batch for g in wl.groups)} matrices x {wl.ns_steps} iterations"),
            "seconds_per_step": round(step_s, 1)}


# ---------------------------------------------------------------------------
# rocprofv3 summaries
# ---------------------------------------------------------------------------

KERNEL_NAMES = (
    ("ns_gemm_kernel<256, 256, 0>", "ns_syrk_xxt"), ("ns_gemm_kernel<256, 256, 1>", "ns_syrk_poly"),
    ("ns_gemm_kernel<256, 256, 2>", "ns_gemm_bx"), ("ns_gemm_kernel<128, 128, 0>", "ns_syrk_xxt [128]"),
    ("ns_gemm_kernel<128, 128, 1>", "ns_syrk_poly [128]"), ("ns_gemm_kernel<128, 128, 2>", "ns_gemm_bx [128]"),
    ("ns_gemm_kernel<256, 128, 0>", "ns_syrk_xxt_slices"), ("ns_gemm_kernel<256, 128, 1>", "ns_syrk_poly_slices"),
    ("momentum_norm_kernel", "momentum_norm"), ("norm_finalize_kernel", "norm_finalize"),
    ("param_update_kernel", "param_update"), ("qk_rowmax_kernel", "qk_rowmax"), ("qk_rowmax_pp_kernel", "qk_rowmax"),
    ("qk_reduce_kernel", "qk_reduce"),
    ("qk_rescale_kernel", "qk_rescale"), ("small_step_kernel", "small_step"), ("thin_gram_kernel", "ns_thin_gram"),
    ("thin_poly_kernel", "ns_thin_poly"), ("thin_bx_kernel", "ns_thin_bx"), ("adamw_kernel", "adamw"),
    ("attn_fwd_kernel", "attn_fwd"), ("mfma_probe_kernel", "mfma_probe"), ("dion_", "dion"))


def short_name(kernel):
    flat = kernel.replace(" ", "")
    for pat, name in KERNEL_NAMES:
        if pat.replace(" ", "") in flat:
            return name
    return "(other: " + kernel[:40] + ")"


def summarize_profile(paths):
    """Per-kernel summary of rocprofv3 CSV output: a kernel trace
    (*_kernel_trace.csv: calls and average / min / max duration), a counter
    collection (*_counter_collection.csv: mean counter value per dispatch) or
    a marker trace (*_marker_api_trace.csv: the library's named host ranges,
    calls and average / min / max host time)."""
    import csv
    from collections import defaultdict
    for path in paths:
        rows = list(csv.DictReader(open(path)))
        if not rows:
            continue
        print(f"# {os.path.basename(path)}")
        if "Function" in rows[0] and "Kernel_Name" not in rows[0]:
            d = defaultdict(list)
            order = []
            for r in rows:
                if r["Function"] not in d:
                    order.append(r["Function"])
                d[r["Function"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            print(f"# {'range':40s} {'calls':>7s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
            for k in order:
                v = d[k]
                print(f"  {k:40s} {len(v):7d} {sum(v) / len(v):10.1f} {min(v):10.1f} {max(v):10.1f}")
        elif "Start_Timestamp" in rows[0]:
            d = defaultdict(list)
            for r in rows:
                d[short_name(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            tot = sum(sum(v) for v in d.values())
            print(f"# {'kernel':28s} {'calls':>7s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>7s}")
            for k, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
                print(f"  {k:28s} {len(v):7d} {sum(v) / len(v):10.1f} {min(v):10.1f} {max(v):10.1f} "
                      f"{100 * sum(v) / tot:7.2f}")
        else:
            d = defaultdict(list)
            for r in rows:
                d[(short_name(r["Kernel_Name"]), r["Counter_Name"])].append(float(r["Counter_Value"]))
            print(f"# {'kernel':28s} {'counter':>12s} {'dispatches':>10s} {'mean_per_dispatch':>18s}")
            for (k, c), v in sorted(d.items()):
                print(f"  {k:28s} {c:>12s} {len(v):10d} {sum(v) / len(v):18.1f}")


def summarize_clock(paths, flops=None):
    """Per-kernel shader clock and MFMA activity from a rocprofv3 counter
    collection of GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES (one run).
    GRBM_GUI_ACTIVE sums the 8 XCDs' busy cycles, so the clock is
    GRBM / 8 / duration; SQ_VALU_MFMA_BUSY_CYCLES counts busy cycles of the
    1024 SIMDs' matrix pipes in units of 8 SIMD-cycles per GRBM cycle summed
    the same way, so the busy share of the matrix pipes is
    MFMA_BUSY / GRBM / 128 (checked against the algorithmic flop of the
    Newton-Schulz products: flop / duration / (clock x 1024 flop/clk x 1024))."""
    import csv
    import statistics
    from collections import defaultdict
    for path in paths:
        per = defaultdict(dict)
        for r in csv.DictReader(open(path)):
            key = (short_name(r["Kernel_Name"]), r["Kernel_Name"][:200], r["Dispatch_Id"])
            per[key][r["Counter_Name"]] = float(r["Counter_Value"])
            per[key]["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        groups = defaultdict(list)
        for (k, full, _), v in per.items():
            if "GRBM_GUI_ACTIVE" in v and "SQ_VALU_MFMA_BUSY_CYCLES" in v and v["dur"] > 0:
                groups[(k, full)].append(v)
        print(f"# {os.path.basename(path)}")
        print(f"# {'kernel':28s} {'launches':>8s} {'median_us':>10s} {'clock_GHz':>10s} {'mfma_busy_%':>12s}")
        for (k, full), vs in sorted(groups.items(), key=lambda kv: -sum(v["dur"] for v in kv[1])):
            if k.startswith("(other"):
                continue
            tag = k
            if k.startswith("ns_") and "<256, 128" in full:
                tag = k + "_slices" if not k.endswith("_slices") else k
            clk = statistics.median(v["GRBM_GUI_ACTIVE"] / 8 / v["dur"] / 1e9 for v in vs)
            busy = statistics.median(v["SQ_VALU_MFMA_BUSY_CYCLES"] / v["GRBM_GUI_ACTIVE"] / 128 * 100 for v in vs)
            dur = statistics.median(v["dur"] for v in vs) * 1e6
            if dur < 50.0:   # the counters' window is longer than a short kernel
                print(f"  {tag:28s} {len(vs):8d} {dur:10.1f} {'-':>10s} {'-':>12s}")
            else:
                print(f"  {tag:28s} {len(vs):8d} {dur:10.1f} {clk:10.3f} {busy:12.1f}")


KERNEL_SOURCES = {
    "ns_": "ns_gemm.hip", "momentum_norm": "elementwise.hip", "param_update": "elementwise.hip",
    "qk_": "qkclip.hip", "small_step": "small.hip", "ns_thin": "thin.hip", "adamw": "adamw.hip",
    "attn_fwd": "attention.hip"}


def summarize_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes=1 << 30):
    """HBM read and write bytes per launch of each of the library's kernels.
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled so that the plain
    1 GiB device copy reads and writes 1 GiB: read = f_r x FETCH_SIZE,
    write = f_w x WRITE_SIZE.  Kernels outside the library are left out."""
    import csv
    import hashlib
    from collections import defaultdict

    def per_kernel(path):
        d = defaultdict(list)
        for r in csv.DictReader(open(path)):
            d[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]) * 1024.0)
        return d

    def copy_value(path):
        vals = [float(r["Counter_Value"]) * 1024.0 for r in csv.DictReader(open(path))
                if "copy" in r["Kernel_Name"].lower()]
        return sum(vals) / len(vals)

    f_r = copy_bytes / copy_value(copy_fetch_csv)
    f_w = copy_bytes / copy_value(copy_write_csv)
    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    print(f"# copy of {copy_bytes / 2**30:.0f} GiB: read bytes = {f_r:.3f} x FETCH_SIZE, "
          f"write bytes = {f_w:.3f} x WRITE_SIZE")
    print(f"# {'kernel':28s} {'launches':>8s} {'read_GB':>9s} {'write_GB':>9s} {'total_GB':>9s}  (mean per launch)")
    out = {}
    for k in sorted(fetch):
        if k.startswith("(other") or k not in write:
            continue
        rd = f_r * sum(fetch[k]) / len(fetch[k])
        wr = f_w * sum(write[k]) / len(write[k])
        print(f"  {k:28s} {len(fetch[k]):8d} {rd / 1e9:9.3f} {wr / 1e9:9.3f} {(rd + wr) / 1e9:9.3f}")
        src = next((v for pfx, v in KERNEL_SOURCES.items() if k.startswith(pfx)), None)
        rel = os.path.join("matrix_orthogonalizing_optimizer_muon_amd", "csrc", src) if src else None
        sha = (hashlib.sha256(open(os.path.join(ROOT, rel), "rb").read()).hexdigest()[:16]
               if rel and os.path.exists(os.path.join(ROOT, rel)) else None)
        out[k] = {"read_bytes": rd, "write_bytes": wr, "total_bytes": rd + wr, "source": rel,
                  "source_sha256_16": sha}
    print("#")
    print("# machine-readable (bench.py uses an entry only while its source hash matches):")
    print("TRAFFIC_JSON " + json.dumps(out, sort_keys=True))


if __name__ == "__main__":
    main()
