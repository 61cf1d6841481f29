"""Host-side logic of bench.py (no GPU): the one-GPU guard, the causal-
adjusted FLOP count against a brute-force count of visible pairs, and the
traffic record's source digest, and which sysfs clock table is read."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle as O
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("length,window", [(1, 0), (7, 0), (100, 0), (100, 1), (100, 37), (50, 50),
                                           (50, 500), (4096, 0), (300, 64)])
def test_visible_pairs_is_the_brute_force_count(length, window):
    if length <= 512:
        want = int(O.visible_mask(np.arange(length), np.arange(length), window).sum())
    else:   # closed form of the causal count, checked against brute force above
        want = length * (length + 1) // 2
    assert bench.visible_pairs(length, window) == want


def test_layer_flop_sums_segments_and_heads():
    w = W.WORKLOADS["thd_16seg_h40kv8_d128"]
    want = sum(4 * w.head_dim * w.num_heads * n * (n + 1) // 2 for n in w.segment_lengths)
    assert bench.layer_flop(w, 0) == want


def test_traffic_record_is_ignored_when_the_kernel_sources_change(tmp_path, monkeypatch):
    digest = bench.kernel_source_digest()
    assert len(digest) == 16 and digest == bench.kernel_source_digest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = dict(kernel_source_digest=digest, fetch_bytes_per_launch=100, write_bytes_per_launch=20)
    (prof / "attn_fused_traffic_x.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: digest)
    assert bench.measured_traffic("x", 1) == 120
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.measured_traffic("x", 1) is None


class _Props:
    pci_domain_id, pci_bus_id, pci_device_id = 0, 0x1c, 0


def _fake_torch(props):
    class _Cuda:
        @staticmethod
        def get_device_properties(dev):
            if props is None:
                raise RuntimeError("no device")
            return props

    class _Torch:
        cuda = _Cuda
    return _Torch


def test_clock_table_is_the_device_s_own(monkeypatch):
    """The clock table is found by the device's PCI address; without one, only
    a single table on the host is taken (several would be ambiguous)."""
    own = "/sys/bus/pci/devices/0000:1c:00.0/pp_dpm_sclk"
    monkeypatch.setattr(bench.os.path, "exists", lambda p: p == own)
    assert bench.sclk_table_path(_fake_torch(_Props), 0) == own
    import glob
    monkeypatch.setattr(bench.os.path, "exists", lambda p: False)
    monkeypatch.setattr(glob, "glob", lambda pat: ["/sys/class/drm/card1/device/pp_dpm_sclk",
                                                   "/sys/class/drm/card0/device/pp_dpm_sclk"])
    assert bench.sclk_table_path(_fake_torch(None), 0) is None
    monkeypatch.setattr(glob, "glob", lambda pat: ["/sys/class/drm/card0/device/pp_dpm_sclk"])
    assert bench.sclk_table_path(_fake_torch(None), 0) == "/sys/class/drm/card0/device/pp_dpm_sclk"


def test_current_clock_is_the_marked_level():
    table = "0: 500Mhz \n1: 1200Mhz \n2: 1844Mhz *\n3: 2400Mhz \n"
    assert bench.current_sclk_mhz(table) == 1844
    assert bench.current_sclk_mhz("0: 500Mhz *\n1: 2400Mhz\n") == 500
    assert bench.current_sclk_mhz("0: 500Mhz\n1: 2400Mhz\n") is None
    assert bench.current_sclk_mhz("") is None
