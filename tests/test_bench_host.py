"""Host-side pieces of the benchmark (no GPU): the one-GPU guard, the algorithmic byte counts
against the packer's sizes, the recorded-traffic lookup, and the committed counter summaries
against the algorithmic bytes."""
import os
import re
import subprocess
import sys

import pytest

import bench
import weight_only_quantized_qgemm_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("fmt,N,K,G", [("int4", 4096, 4096, 128), ("int4", 11008, 4096, 32), ("int2", 4096, 4096, 128),
                                       ("nf4", 4096, 4096, 64), ("fp8", 10240, 5120, 0), ("fp8h", 10240, 5120, 0),
                                       ("fp4", 8192, 8192, 16)])
def test_weight_bytes_are_the_packed_sizes(fmt, N, K, G):
    # the algorithmic bytes behind every GB/s figure are exactly what the packer produces
    p = q.problem(1, N, K, fmt, group_size=G if fmt in q.GROUP_SCALED else None)
    wb, sb = q.packed_sizes(p)
    assert bench.weight_bytes(fmt, N, K, G) == wb + sb


def test_recorded_traffic_follows_the_kernel_sources(monkeypatch):
    t = bench.recorded_traffic()
    assert t is None or (isinstance(t, int) and t > bench.weight_bytes("int4", 4096, 4096, 128))
    # a different decode source hash makes the recorded counters stale
    monkeypatch.setattr(bench, "kernel_sha", lambda kind: "0" * 16)
    assert bench.recorded_traffic() is None


def test_measurement_library_loads_and_sizes_the_stream_grid():
    # the streaming-read and host-timing helpers live in their own library next to libqgemm.so
    lib = bench._probe_lib()
    for name in ("qgemm_probe_stream", "qgemm_probe_stream_groups", "qgemm_probe_host_ns"):
        assert hasattr(lib, name)
    # 8 MiB of 16-byte chunks with 4 loads per thread of 512 threads: 256 workgroups
    assert lib.qgemm_probe_stream_groups((8 << 20) // 16, 4) == 256
    assert lib.qgemm_probe_stream_groups(1, 8) == 1
    # bad arguments are refused on the host, before any launch (no GPU needed)
    assert lib.qgemm_probe_stream(None, 1024, None, 0, None, 4, None) == -1
    assert lib.qgemm_probe_stream(16, 1000, None, 0, 16, 4, None) == -1       # not a multiple of 16
    assert lib.qgemm_probe_stream(16, 1024, None, 0, 16, 3, None) == -1       # U not offered


def test_committed_counters_cover_the_algorithmic_bytes():
    # bench sanity on the committed counter summaries: every profiled launch fetched at least
    # the bytes it must read (weights and scales; for the prefill also A) and wrote at least its
    # output, and the decode weight bytes there are the packer's sizes
    txt = open(os.path.join(ROOT, "profiles", "qgemm_decode_int4_traffic.txt")).read()
    rows = re.findall(r"M=(\d+)\s+N=(\d+)\s+K=(\d+).*->\s+([\d.]+) MB\s+\(weights\s+([\d.]+) MB", txt)
    assert len(rows) == 4
    for M, N, K, measured, weights in rows:
        assert float(measured) >= float(weights)
        assert abs(float(weights) * 1e6 - bench.weight_bytes("int4", int(N), int(K), 128)) < 1e3
    txt = open(os.path.join(ROOT, "profiles", "qgemm_prefill_bench.txt")).read()
    rows = re.findall(r"HBM fetch\s+([\d.]+) MB \(algorithmic A \+ weights\s+([\d.]+) MB\), "
                      r"write\s+([\d.]+) MB \(output\s+([\d.]+) MB\)", txt)
    assert len(rows) >= 5
    for fetch, algorithmic, write, output in rows:
        assert float(fetch) >= float(algorithmic) and float(write) >= float(output)
