"""Host logic of the benchmark (CPU only): the algorithmic work it divides
by, the bytes it counts for the HBM passes, the traffic summary it reads
from rocprofv3 counter files, the source-hash gate on stored traffic, and the
one-GPU refusal.

The flop totals per step are pinned to figures computed separately from the
Newton-Schulz cost paragraph of "Muon and MuonClip: orthogonalised updates
for LLM training" (section 2: 2(2nm^2 + m^3) per iteration of a wide m x n
matrix, here summed over every matrix of each workload for 5 iterations):
dense 1.05e-4, 3.350, 499.42, 131.94 and 48.40 TFLOP; with the two symmetric
products counted on their upper triangles 7.36e-5, 2.363, 353.86, 94.85 and
32.62 TFLOP."""
import csv
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synthetic import generators as gen  # noqa: E402

DENSE = {1: 1.048576e-4, 2: 3.35007, 3: 499.4188, 4: 131.9414, 5: 48.40428}
ALGORITHMIC = {1: 7.364608e-5, 2: 2.362714, 3: 353.8559, 4: 94.85100, 5: 32.62248}


def per_step(idx, fn):
    wl = gen.workload(idx)
    total = 0
    for g in wl.groups:
        m, n = min(g.rows, g.cols), max(g.rows, g.cols)
        f = fn(m, n)
        total += g.batch * wl.ns_steps * (sum(f.values()) if isinstance(f, dict) else f)
    return total / 1e12


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_flop_model_per_step(idx):
    dense = per_step(idx, bench.ns_flops_dense)
    alg = per_step(idx, bench.ns_flops)
    assert abs(dense / DENSE[idx] - 1) < 1e-5
    assert abs(alg / ALGORITHMIC[idx] - 1) < 1e-5
    # the symmetric products save at most half of their own work
    assert 0.5 * dense < alg < dense


def test_flop_model_terms():
    m, n = 3, 5
    f = bench.ns_flops(m, n)
    # X X^T: m(m+1)/2 dot products of length n, 2 flop each; A A^T: the same
    # with length m; B X: m n dot products of length m
    assert f["ns_syrk_xxt"] == 2 * (m * (m + 1) // 2) * n
    assert f["ns_syrk_poly"] == 2 * (m * (m + 1) // 2) * m
    assert f["ns_gemm_bx"] == 2 * m * n * m


def test_hbm_pass_bytes():
    elem = 10 ** 8
    prof = {"momentum_norm": (2.0, 4), "param_update": (1.0, 2)}   # total ms, launches
    out = bench.hbm_passes(prof, elem, None)
    mom, upd = out["momentum_norm"], out["param_update"]
    assert mom["bytes"] == 12 * elem and mom["bytes_moved"] == 14 * elem
    assert upd["bytes"] == 6 * elem and upd["bytes_moved"] == 6 * elem
    assert mom["avg_us"] == 500.0 and upd["avg_us"] == 500.0
    assert mom["GBs"] == pytest.approx(12 * elem / 500e-6 / 1e9)
    assert mom["frac"] == pytest.approx(mom["GBs"] / 8000.0, abs=1e-4)
    assert mom["traffic"] is None
    bench.attach_hbm_probe(out, {"mix_6r_8w_GBs": mom["GBs_moved"] * 2, "mix_4r_2w_GBs": upd["GBs_moved"]})
    assert mom["frac_of_stream_probe"] == 0.5 and upd["frac_of_stream_probe"] == 1.0


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
        w.writeheader()
        for name, v in rows:
            w.writerow({"Kernel_Name": name, "Counter_Value": v})


def test_traffic_summary_scales_by_the_copy(tmp_path, capsys):
    gib_kib = float(1 << 20)   # 1 GiB in KiB
    # the copy reads half its bytes as FETCH_SIZE (64-byte requests counted
    # as 32) and writes all of them as WRITE_SIZE
    write_csv(tmp_path / "cf.csv", [("copy_kernel", gib_kib / 2)])
    write_csv(tmp_path / "cw.csv", [("copy_kernel", gib_kib)])
    bx = "muon::ns_gemm_kernel<256, 256, 2>(muon::GemmLaunch)"
    write_csv(tmp_path / "f.csv", [(bx, 1000.0), (bx, 3000.0), ("void at::native::foo", 5.0)])
    write_csv(tmp_path / "w.csv", [(bx, 10.0), (bx, 30.0), ("void at::native::foo", 5.0)])
    bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                            str(tmp_path / "cw.csv"))
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("TRAFFIC_JSON ")][0]
    data = json.loads(line[len("TRAFFIC_JSON "):])
    assert set(data) == {"ns_gemm_bx"}                    # other kernels left out
    e = data["ns_gemm_bx"]
    assert e["read_bytes"] == pytest.approx(2 * 2000.0 * 1024)   # mean of the launches, x 2
    assert e["write_bytes"] == pytest.approx(20.0 * 1024)
    src = os.path.join(ROOT, e["source"])
    assert e["source_sha256_16"] == hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def test_stored_traffic_is_used_only_while_the_source_matches(tmp_path):
    src = "matrix_orthogonalizing_optimizer_muon_amd/csrc/ns_gemm.hip"
    good = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()[:16]
    data = {"ns_gemm_bx": {"source": src, "source_sha256_16": good, "total_bytes": 123.0},
            "ns_syrk_xxt": {"source": src, "source_sha256_16": "0" * 16, "total_bytes": 456.0},
            "norm_finalize": {"source": None, "source_sha256_16": None, "total_bytes": 7.0}}
    p = tmp_path / "traffic.txt"
    p.write_text("# summary\nTRAFFIC_JSON " + json.dumps(data) + "\n")
    assert bench.measured_traffic(str(p)) == {"ns_gemm_bx": 123.0}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
