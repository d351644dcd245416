"""bench.py's host logic, without a GPU: the single-GPU contract, the stored-traffic lookup
(reported only while the kernel sources hash to the digest the counters were taken on) and
the per-kernel trace summary (each kernel's last K dispatches)."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def _write_traffic(tmp_path, kernel, workload, hbm, sha):
    prof = tmp_path / "profiles"
    prof.mkdir(exist_ok=True)
    (prof / ("%s_%s_traffic.md" % (kernel, workload))).write_text(
        "# header\n\nprose line: with a colon\n\n- hbm_bytes_per_launch: %d\n"
        "- algorithmic_bytes_per_launch: 1000\n- source_sha256: `%s`\n" % (hbm, sha))


def test_stored_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "ab" * 32)
    _write_traffic(tmp_path, "attention_kernel", "wl", 123456789, "ab" * 32)
    assert bench.stored_traffic("wl", "attention_kernel") == 123456789
    # counters taken on other sources are not reported
    _write_traffic(tmp_path, "attention_kernel", "wl", 123456789, "cd" * 32)
    assert bench.stored_traffic("wl", "attention_kernel") is None
    # no summary at all
    assert bench.stored_traffic("other", "attention_kernel") is None


def test_committed_traffic_summaries_are_parseable():
    """Every committed traffic summary carries the three values bench.py reads."""
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith("_traffic.md")]
    assert names
    for n in names:
        vals = {}
        for line in open(os.path.join(prof, n)):
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
        assert int(vals["hbm_bytes_per_launch"]) > 0, n
        assert int(vals["algorithmic_bytes_per_launch"]) > 0, n
        assert len(vals["source_sha256"]) == 64, n


def test_kernel_source_digest_covers_the_hip_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "bit_kv_cache_pack_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("kernel a")
    (csrc / "b.cuh").write_text("helpers")
    (csrc / "notes.txt").write_text("not a source")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_source_digest()
    (csrc / "notes.txt").write_text("changed, still not a source")
    assert bench.kernel_source_digest() == d0
    (csrc / "b.cuh").write_text("helpers, changed")
    assert bench.kernel_source_digest() != d0


def test_trace_summary_keeps_each_kernels_last_dispatches(tmp_path, capsys):
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    # 3 warm-up dispatches of 50 us, then 4 timed ones of 10, 20, 30, 40 us; a second kernel
    for dur in [50, 50, 50, 10, 20, 30, 40]:
        rows.append('"void kvq::(anonymous namespace)::attention_kernel<128, true, false, false>'
                    '(kvq::AttnParams)",%d,%d' % (t, t + dur * 1000))
        t += 100000
        rows.append("_ZN3kvq12_GLOBAL__N_118quant_split_kernelIDF16bLi128ELi2EEEvNS_17QuantAppendParamsE,%d,%d"
                    % (t, t + 5000))
        t += 100000
    path = tmp_path / "trace.csv"
    path.write_text("\n".join(rows) + "\n")
    bench.trace_summary(str(path), 4)
    out = capsys.readouterr().out.splitlines()
    att = [l for l in out if "attention_kernel<128, true, false, false>" in l]
    assert len(att) == 1
    cells = [c.strip() for c in att[0].strip("|").split("|")]
    assert cells[1] == "4"
    assert float(cells[2]) == np.mean([10, 20, 30, 40])
    assert float(cells[3]) == np.median([10, 20, 30, 40])
    assert (float(cells[4]), float(cells[5])) == (10.0, 40.0)
    q = [l for l in out if "quant_split_kernel" in l]
    assert len(q) == 1 and "| 4 | 5.0 | 5.0 | 5.0 | 5.0 |" in q[0]


def test_host_cpu_names_the_generation():
    h = bench.host_cpu()
    for k in ("cpu_model", "cpu_vendor", "cpu_family", "cpu_model_number", "nproc", "OMP_NUM_THREADS"):
        assert k in h
    assert h["nproc"] == os.cpu_count()
