"""bench.py's host side on the CPU: the one-GPU guard, the kernel-source
digest that ties counter summaries to the code they were taken on, the
reading of a counter summary, and the host baseline leg.  Nothing here
touches a GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no result line


def _fake_tree(tmp_path, text):
    csrc = tmp_path / "ternary_group_scaled_q1_amd" / "csrc"
    csrc.mkdir(parents=True, exist_ok=True)
    (csrc / "k.hip").write_text(text)
    (csrc / "notes.txt").write_text("not a source file")
    return tmp_path


def test_source_digest_ignores_comments_only(tmp_path, monkeypatch):
    code = "int f(int a) {\n  return a + 1;\n}\n"
    monkeypatch.setattr(bench, "ROOT", str(_fake_tree(tmp_path, code)))
    d0 = bench._source_digest()
    _fake_tree(tmp_path, "// a header comment\n\nint f(int a) {  // trailing note\n\n  return a + 1;\n}\n")
    assert bench._source_digest() == d0
    _fake_tree(tmp_path, "int f(int a) {\n  return a + 2;\n}\n")
    assert bench._source_digest() != d0
    _fake_tree(tmp_path, code)
    (tmp_path / "ternary_group_scaled_q1_amd" / "csrc" / "notes.txt").write_text("changed")
    assert bench._source_digest() == d0  # only .hip / .hpp / .cpp count
    from ternary_group_scaled_q1_amd import build as bld
    monkeypatch.setitem(bld.EXTRA_FLAGS, "k.hip", ["-mllvm", "-some-scheduler-flag"])
    assert bench._source_digest() != d0  # the flags a source is built with count too


def _summary(tmp_path, digest, sweep="tq2_M16", fetch="1000", write="200"):
    lines = ["# a counter summary", "", "| kernel | x |", "|---|---|",
             "    a command line: with a colon", f"source_sha256: {digest}", f"sweep: {sweep}"]
    if fetch is not None:
        lines.append(f"fetch_bytes_per_launch: {fetch}")
    if write is not None:
        lines.append(f"write_bytes_per_launch: {write}")
    p = tmp_path / "traffic.txt"
    p.write_text("\n".join(lines) + "\n")
    return str(p)


def test_measured_traffic_reads_only_a_current_summary(tmp_path, monkeypatch):
    digest = bench._source_digest()
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, digest))
    assert bench.measured_traffic(("tq2", 16)) == (1200, 1000)
    assert bench.measured_traffic(("q1", 16)) == (None, None)  # another sweep
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, "0" * 64))
    assert bench.measured_traffic(("tq2", 16)) == (None, None)  # kernels changed since
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, digest, write=None))
    assert bench.measured_traffic(("tq2", 16)) == (None, 1000)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic(("tq2", 16)) == (None, None)


def test_measured_traffic_per_sweep_lines(tmp_path):
    digest = bench._source_digest()
    p = tmp_path / "traffic.txt"
    p.write_text("\n".join(["# summary", f"source_sha256: {digest}",
                             "fetch_bytes_per_launch.tq2_M16: 1000", "write_bytes_per_launch.tq2_M16: 200",
                             "fetch_bytes_per_launch.q1_M16: 700", "write_bytes_per_launch.q1_M16: 100"]) + "\n")
    old = bench.TRAFFIC_FILE
    bench.TRAFFIC_FILE = str(p)
    try:
        assert bench.measured_traffic(("tq2", 16)) == (1200, 1000)
        assert bench.measured_traffic(("q1", 16)) == (800, 700)
        assert bench.measured_traffic(("q1", 1)) == (None, None)  # not measured
    finally:
        bench.TRAFFIC_FILE = old


def test_committed_summary_has_the_machine_readable_lines():
    keys = {}
    with open(bench.TRAFFIC_FILE) as f:
        for ln in f:
            if ":" in ln and not ln.startswith(("#", "|", " ")):
                k, v = ln.split(":", 1)
                keys[k.strip()] = v.strip()
    assert len(keys["source_sha256"]) == 64
    sweeps = [k.split(".", 1)[1] for k in keys if k.startswith("fetch_bytes_per_launch.")]
    assert sweeps and set(sweeps) <= {f"{f}_M{m}" for f in ("q1", "tq2") for m in (1, 16)}
    for sw in sweeps:
        assert int(keys[f"fetch_bytes_per_launch.{sw}"]) > 0 and int(keys[f"write_bytes_per_launch.{sw}"]) > 0


def test_cpu_baseline_leg_reports_the_oracle():
    cases = [("q1 GEMV 24576x4096 M=1", "q1", 24576, 4096, 1, "f16", 32),
             ("tq5 GEMM 512x5120x17408", "tq5", 5120, 17408, 16, "bf16", 16)]
    r = bench.cpu_baseline(0.01, cases=cases)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["nproc"] >= 1 and r["cpu_model"]
    for label, *_ in cases:
        e = r["per_shape"][label]
        for tag in ("1", "all"):
            assert e[f"full_shape_s_{tag}"] > 0 and e[f"weights_per_s_{tag}"] > 0 and e[f"tok_s_{tag}"] > 0


def test_bench_shape_table_covers_the_workloads():
    """Single-launch timings cover the 8B-class q1 decode shapes, the
    27B-class tq2 shapes at 1, 4 and 8 tokens, and every sweep launch."""
    labels = [s[0] for s in bench.SHAPES]
    for N, K in ((24576, 4096), (4096, 12288), (151936, 4096)):
        assert f"q1 {N}x{K} M=1 f16" in labels
    for N, K in ((34816, 5120), (5120, 17408)):
        for m in (1, 4, 8):
            assert f"tq2 {N}x{K} M={m} bf16" in labels
    assert sum("sweep" in lab for lab in labels) == 20
    assert bench.POOL_BYTES >= 1 << 30
