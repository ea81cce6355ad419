"""Host logic of bench.py (no GPU): the FLOP and pair counts behind every
reported rate, the HBM-traffic summary built from counter CSVs and the rule
that a traffic figure is only reported for the workload and kernel sources it
was measured on, and the one-GPU guard."""
import csv
import importlib.util
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def brute_pairs(N, mask, window):
    n = 0
    for i in range(N):
        for j in range(N):
            if mask == "causal" and j > i:
                continue
            if mask == "local" and abs(i - j) > window:
                continue
            n += 1
    return n


@pytest.mark.parametrize("N", [1, 2, 7, 33, 64])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("local", 0), ("local", 1),
                                         ("local", 5), ("local", 40), ("local", 1000)])
def test_pair_count_matches_brute_force(bench, N, mask, window):
    assert bench.attn_pairs(N, mask, window) == brute_pairs(N, mask, window)


def _w(B, H, N, d, mask="none", window=0, dtype="bf16"):
    return types.SimpleNamespace(shape=(B, H, N, d), mask=mask, window=window, dtype=dtype)


def test_flop_and_byte_counts(bench):
    w = _w(2, 16, 4096, 128)
    assert bench.fwd_flops(w) == 4.0 * 2 * 16 * 4096 * 4096 * 128
    assert bench.fwd_flops(_w(2, 16, 4096, 128, "causal")) == bench.fwd_flops(w) / 2
    assert bench.bwd_flops(w) == 2.5 * bench.fwd_flops(w)
    band = _w(1, 32, 16384, 128, "local", 128)
    assert bench.fwd_flops(band) == 4.0 * 32 * (16384 * 257 - 128 * 129) * 128
    # bf16: Q, K, V in and O out at 2 bytes, LSE at 4; backward 8 tensors + LSE
    assert bench.fwd_bytes(w) == 4 * 2 * 16 * 4096 * 128 * 2 + 2 * 16 * 4096 * 4
    assert bench.bwd_bytes(w) == 8 * 2 * 16 * 4096 * 128 * 2 + 2 * 16 * 4096 * 4


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for disp, name, val in rows:
            wr.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": val})


def test_summarize_pmc_scales_and_tags_the_workload(bench, tmp_path):
    d = tmp_path
    # the 1 MiB calibration copy reads half its bytes by FETCH_SIZE and all by WRITE_SIZE
    _counter_csv(d / "copy_fetch_counter_collection.csv", "FETCH_SIZE", [(1, "copyBuffer", 512.0)])
    _counter_csv(d / "copy_write_counter_collection.csv", "WRITE_SIZE", [(1, "copyBuffer", 1024.0)])
    # two dispatches each; the per-dispatch mean is used; several counter
    # instances of one dispatch add up
    _counter_csv(d / "fetch_counter_collection.csv", "FETCH_SIZE", [
        (1, "void fa::bwd_dq_bf16_kernel<128>(fa::BwdArgs)", 60.0),
        (1, "void fa::bwd_dq_bf16_kernel<128>(fa::BwdArgs)", 40.0),
        (3, "void fa::bwd_dq_bf16_kernel<128>(fa::BwdArgs)", 100.0),
        (2, "void fa::bwd_dkdv2_bf16_kernel<128>(fa::BwdArgs)", 50.0),
        (4, "void fa::bwd_dkdv2_bf16_kernel<128>(fa::BwdArgs)", 150.0),
        (5, "void fa::fwd_bf16_kernel<128>(fa::FwdArgs)", 10.0),
        (6, "some_other_kernel", 999.0)])
    _counter_csv(d / "write_counter_collection.csv", "WRITE_SIZE", [
        (1, "void fa::bwd_dq_bf16_kernel<128>(fa::BwdArgs)", 8.0),
        (2, "void fa::bwd_dkdv2_bf16_kernel<128>(fa::BwdArgs)", 16.0),
        (5, "void fa::fwd_bf16_kernel<128>(fa::FwdArgs)", 4.0)])
    text = bench.summarize_pmc(str(d), 1, "some_workload")
    meta = json.loads(text.split(bench.TRAFFIC_TAG)[1].split("-->")[0])
    assert meta["workload"] == "some_workload"
    assert meta["fetch_factor"] == 2.0 and meta["write_factor"] == 1.0
    # fa_bwd: (100 + 100) KiB read x 2, (8 + 16) KiB written
    assert meta["units"]["fa_bwd"] == {"read_bytes": 200 * 1024 * 2, "write_bytes": 24 * 1024}
    assert meta["units"]["fa_fwd"] == {"read_bytes": 10 * 1024 * 2, "write_bytes": 4 * 1024}
    assert "some_other_kernel" not in text


def test_traffic_only_for_same_workload_and_sources(bench, tmp_path):
    sha = bench.kernel_source_sha()
    def summary(name, sha_, workload):
        meta = {"source_sha": sha_, "workload": workload, "fetch_factor": 2.0, "write_factor": 1.0,
                "units": {"fa_bwd": {"read_bytes": 300, "write_bytes": 100}}}
        (tmp_path / name).write_text(f"# x\n\n<!-- {bench.TRAFFIC_TAG} {json.dumps(meta)} -->\n")
    summary("a.md", sha, "wl_a")
    summary("b.md", "0" * 16, "wl_b")  # taken on other kernel sources
    assert bench.load_traffic("fa_bwd", "wl_a", str(tmp_path))[0] == 400
    assert bench.load_traffic("fa_bwd", "wl_b", str(tmp_path)) == (None, None)
    assert bench.load_traffic("fa_bwd", "wl_c", str(tmp_path)) == (None, None)
    assert bench.load_traffic("fa_fwd", "wl_a", str(tmp_path)) == (None, None)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU only" in r.stderr


def test_cpu_baseline_keys(bench):
    """The CPU-baseline leg on a tiny workload of the same recipe: dense and
    tiled forward and dense backward timed per slice, the rate from the dense
    pair, the thread count and the CPU model stated."""
    from exact_tiled_attention_fwd_amd.synth import Workload, make_inputs
    w = Workload("tiny_causal_bwd", 1, 3, 70, 16, "bf16", "causal", seed=1, backward=True)
    inp = make_inputs(w)
    r = bench.cpu_baseline(w, inp, True, target_s=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert r["cores"] == bench.omp_threads() >= 1
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    for key in ("dense_fwd_s", "tiled_fwd_s", "dense_bwd_s"):
        assert r[key] >= 0
    assert r["sample"].startswith("1 of 3 (b,h) slices [1,1,70,16]")
    ff = bench.fwd_flops(type(w)(**{**w.__dict__, "B": 1, "H": 1}))
    fb = 2.5 * ff
    assert abs(r["value"] - (ff + fb) / (r["dense_fwd_s"] + r["dense_bwd_s"]) / 1e12) <= \
        1e-6 + 1e-2 * r["value"]


def test_oracle_all_covers_every_workload(bench):
    """bench.py --oracle-all: one row per workload of the statement, in
    order, each with at least one slice timed and the backward only on c5."""
    text = bench.oracle_all(target_s=0.0)
    rows = [ln for ln in text.splitlines() if ln.startswith("| c")]
    assert [r.split("|")[1].strip() for r in rows] == ["c1", "c2", "c3", "c4", "c5"]
    for r, name in zip(rows, bench.STATEMENT_WORKLOADS):
        cells = [c.strip() for c in r.split("|")[1:-1]]
        assert cells[1] == f"`{name}`" and cells[2].startswith("1 of ")
        assert float(cells[3]) > 0 and float(cells[5].split()[0]) > 0
        assert (cells[7] != "—") == (name == "bf16_causal_bwd_b2h16_n4096_d128")
    assert f"{bench.omp_threads()} OpenMP threads" in text
