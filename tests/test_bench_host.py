"""Host-side logic of bench.py (no GPU): the one-GPU guard, the flop counts
the metric uses, the settle-call bounds and the rule that a stored traffic
measurement is reported only while the measured kernels' sources are
unchanged."""

import json
import os
import subprocess
import sys

import bench
import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    """--gpus above 1 ends with a JSON error line and exit status 2, before
    anything touches a GPU."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "error" in line and line["n_gpus"] == 2


def test_forward_flops():
    """4·B·H·N²·d for the forward, halved with the causal mask; the step is
    the forward plus the backward at 2.5 times it."""
    w = si.WORKLOADS["train_causal"]
    assert (w.B, w.H, w.N, w.d, w.causal) == (4, 16, 4096, 128, True)
    assert bench.fwd_flops(w) == 4 * 4 * 16 * 4096 * 4096 * 128 / 2
    nc = si.WORKLOADS["short_noncausal"]
    assert bench.fwd_flops(nc) == 4.0 * nc.B * nc.H * nc.N * nc.N * nc.d


def test_settle_calls_bounds():
    assert bench.settle_calls(1e18) == 3          # very large calls: at least 3
    assert bench.settle_calls(1.0) == 2000        # tiny calls: at most 2000
    assert bench.settle_calls(1e12) == 100        # 0.1 s at 1 PFLOP/s


def test_stored_traffic_follows_the_sources(tmp_path, monkeypatch):
    """A stored measurement is returned only for its workload and while the
    SHA-256 it carries matches the current kernel sources; a missing file,
    another hash or another workload give None."""
    t = {"workload": "train_causal", "source_sha256": bench.kernel_source_hash(),
         "bytes_per_launch": {"fa_fwd": 1, "fa_bwd": 2}}
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.stored_traffic("train_causal") is None
    f.write_text(json.dumps(t))
    assert bench.stored_traffic("train_causal") == t
    assert bench.stored_traffic("long_causal") is None
    f.write_text(json.dumps(dict(t, source_sha256="0" * 64)))
    assert bench.stored_traffic("train_causal") is None
    f.write_text("not json")
    assert bench.stored_traffic("train_causal") is None


def test_source_hash_covers_the_measured_kernels(tmp_path, monkeypatch):
    """Every file the hash covers exists, and changing one byte of any of
    them changes the hash."""
    import shutil

    csrc = os.path.join(ROOT, "exact_tiled_attention_37_amd", "csrc")
    assert {"fa_fwd.hip", "fa_bwd.hip", "fa_common.hpp"} <= set(bench.TRAFFIC_SOURCES)
    copy = tmp_path / "exact_tiled_attention_37_amd" / "csrc"
    copy.mkdir(parents=True)
    for name in bench.TRAFFIC_SOURCES:
        shutil.copy(os.path.join(csrc, name), copy / name)
    base = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash() == base
    for name in bench.TRAFFIC_SOURCES:
        data = (copy / name).read_bytes()
        (copy / name).write_bytes(data[:-1] + bytes([data[-1] ^ 1]))
        assert bench.kernel_source_hash() != base, name
        (copy / name).write_bytes(data)
    assert bench.kernel_source_hash() == base
