"""Host-side behaviour of bench.py that needs no GPU: the one-GPU contract and the rule
that stored HBM-traffic counts are reported only for the kernel source they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fake_tree(tmp_path, source_text):
    for f in bench.KERNEL_SOURCES:
        p = tmp_path / f
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text(source_text)
    (tmp_path / "profiles").mkdir(exist_ok=True)


def test_traffic_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _fake_tree(tmp_path, "kernel v1")
    h1 = bench.kernel_source_hash()
    entry = {"bytes_per_launch": 123456.0}
    (tmp_path / "profiles" / "traffic.json").write_text(
        json.dumps({"source_sha256": h1, "shapes": {"shape_a": entry}}))
    assert bench.load_traffic("shape_a") == 123456.0
    assert bench.load_traffic("shape_b") is None
    _fake_tree(tmp_path, "kernel v2")                  # the kernel changed since
    assert bench.kernel_source_hash() != h1
    assert bench.load_traffic("shape_a") is None


def test_traffic_absent_or_unreadable(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _fake_tree(tmp_path, "kernel")
    assert bench.load_traffic("shape_a") is None
    (tmp_path / "profiles" / "traffic.json").write_text("{not json")
    assert bench.load_traffic("shape_a") is None


def test_trace_summary_charges_reductions_to_their_call(tmp_path, capsys):
    """A kernel trace of two steps of the decode family: each call is one GEMM dispatch
    (staged or B-streaming), some followed by a split-K reduction; other kernels are
    ignored.  The first step's calls follow a fill kernel (the cache flush): cold; the
    second step's do not: warm."""
    from moe_grouped_gemm_block_amd import synth
    names = [x["name"] for x in synth.workload_shapes(2)]
    lines = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    expect = {k: ({n: [] for n in names}, {n: [] for n in names}) for k in ("cold", "warm")}
    for step in range(2):
        kind_t = "cold" if step == 0 else "warm"
        for i, n in enumerate(names):
            if step == 0:
                lines.append(f"\"vectorized_elementwise_kernel<FillFunctor<int> >\",{t},{t + 90}")
                t += 100
            kind = "fp8bs_stream_kernel<64>" if i % 2 else "fp8bs_gemm_kernel<256>"
            dur = 1000 * (i + 1) + step * 10
            lines.append(f"\"{kind}\",{t},{t + dur}")
            expect[kind_t][0][n].append(dur / 1e3)
            t += dur + 50
            lines.append(f"\"spin_kernel\",{t},{t + 7}")
            t += 100
            if i % 3 == 0:
                lines.append(f"\"fp8bs_splitk_reduce<64>\",{t},{t + 300 + i}")
                expect[kind_t][1][n].append((300 + i) / 1e3)
                t += 400
    (tmp_path / "run").mkdir()
    (tmp_path / "run" / "kt_kernel_trace.csv").write_text("\n".join(lines) + "\n")
    bench.summarize_trace(str(tmp_path), 2)
    out = json.loads(capsys.readouterr().out)
    for kind_t in ("cold", "warm"):
        for n in names:
            g, r = expect[kind_t][0][n], expect[kind_t][1][n]
            rec = out[n][kind_t]
            assert rec["dispatches"] == 1
            assert abs(rec["avg_us"] - sum(g)) < 1e-9
            assert rec["reduce_dispatches"] == len(r)
            ravg = sum(r) / len(r) if r else 0.0
            assert abs(rec["call_avg_us"] - (sum(g) + ravg * len(r))) < 1e-9


def test_family_list_and_cpu_model():
    assert bench.parse_families("none", 3) == []
    assert bench.parse_families("0,1,3,2,1", 3) == [0, 1, 2]
    with pytest.raises(SystemExit):
        bench.parse_families("9", 3)
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_input_hash_covers_group_data():
    from moe_grouped_gemm_block_amd import synth
    p = synth.make_contiguous(2, 64, 128, seed=5, total_rows=200)
    h = bench.input_sha256(p)
    assert h == bench.input_sha256(p)
    p.layout = p.layout.copy()
    p.layout[0] = -1
    assert bench.input_sha256(p) != h


def test_mfma_busy_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _fake_tree(tmp_path, "kernel v1")
    h1 = bench.kernel_source_hash()
    entry = {"mfma_busy_frac": 0.42, "sclk_ghz": 2.05}
    (tmp_path / "profiles" / "mfma.json").write_text(
        json.dumps({"source_sha256": h1, "shapes": {"shape_a": entry}}))
    assert bench.load_mfma_busy("shape_a") == {"busy_frac": 0.42, "sclk_ghz": 2.05}
    assert bench.load_mfma_busy("shape_b") is None
    _fake_tree(tmp_path, "kernel v2")
    assert bench.load_mfma_busy("shape_a") is None
