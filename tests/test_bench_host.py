"""Host-side logic of bench.py: the one-GPU guard, the kernel-source hash and
the lookup of counter-measured traffic.  No GPU is touched."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, env=e, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash_covers_each_format():
    hashes = {f: bench.kernel_source_hash(f) for f in bench.GEMM_SOURCES}
    for h in hashes.values():
        assert re.fullmatch(r"[0-9a-f]{16}", h)
    # every format has its own set: the generic tile kernel plus, for Q6_K
    # and two-bit ternary, the few-token ring kernel (and for Q6_K its
    # matrix-vector kernel), for base-3 ternary its register-unpack tile
    # kernel; Q4_K its own kernels
    assert len(set(hashes.values())) == len(hashes)
    assert "kq_gemm_tq.hip" in bench.GEMM_SOURCES["tq"] and "kq_tile.hpp" in bench.GEMM_SOURCES["q4_k"]
    for f in ("q6_k", "tq2"):
        assert "kq_gemm_ring.hip" in bench.GEMM_SOURCES[f]
    assert "kq_gemv.hip" in bench.GEMM_SOURCES["q6_k"] and "kq_gemv.hip" not in bench.GEMM_SOURCES["tq2"]
    for srcs in bench.GEMM_SOURCES.values():
        for s in srcs:
            assert os.path.exists(os.path.join(bench.CSRC, s)), s


def _fake_profiles(tmp_path, name, sha, nbytes):
    d = tmp_path / "profiles"
    d.mkdir(exist_ok=True)
    (d / name).write_text(f"# traffic\n\nkernel_source_sha256_16: {sha}\n"
                          f"hbm_bytes_per_launch: {nbytes}\n")


def test_measured_traffic_needs_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    cur = bench.kernel_source_hash("q4_k")
    _fake_profiles(tmp_path, "gemm_q4k_ffn_up_q4k_2048_traffic.md", cur, "1.25e+08")
    _fake_profiles(tmp_path, "gemm_q4k_ring_ffn_up_q4k_64_traffic.md", "0" * 16, "3.4e+07")
    assert bench.measured_traffic("ffn_up_q4k_2048", "q4_k") == pytest.approx(1.25e8)
    # taken on another kernel source: not reported
    assert bench.measured_traffic("ffn_up_q4k_64", "q4_k") is None
    # no file for the workload, or a file under another format's hash
    assert bench.measured_traffic("ffn_up_q4k_1", "q4_k") is None
    assert bench.measured_traffic("ffn_up_q4k_2048", "q6_k") is None


def test_measured_traffic_without_profiles(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("ffn_up_q4k_2048", "q4_k") is None


def test_committed_traffic_summaries_are_well_formed():
    pdir = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(pdir) if n.endswith("_traffic.md")]
    assert names, "no traffic summaries committed"
    for n in names:
        text = open(os.path.join(pdir, n)).read()
        h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
        b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
        assert h and len(h.group(1)) == 16, n
        assert b and float(b.group(1)) > 0, n
        assert "rocprofv3" in text, f"{n} does not give the command that made it"
