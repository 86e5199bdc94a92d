"""bench.py's host logic (no GPU): the one-GPU refusal and the gating of the
counted traffic figure on the kernel sources it was measured with."""
import hashlib
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HASHED = ("step_kernels.hip", "elemops.hpp", "launch.hpp")
PROFILE = os.path.join("profiles", "ring_rs_step_p8_fp32_64Mi_hbm_traffic.md")


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)


def _tree(tmp_path, edit=None):
    """A copy of the hashed kernel sources and the traffic summary under tmp_path."""
    csrc = tmp_path / "allreduce_reduction_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in HASHED:
        shutil.copy(os.path.join(ROOT, "allreduce_reduction_amd", "csrc", f), csrc / f)
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, PROFILE), tmp_path / PROFILE)
    if edit:
        with open(csrc / edit, "a", encoding="utf-8") as fh:
            fh.write("\n// edited\n")
    return tmp_path


def test_traffic_is_reported_for_the_measured_sources(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    src = b"".join(open(os.path.join(ROOT, "allreduce_reduction_amd", "csrc", f), "rb").read() for f in HASHED)
    text = open(os.path.join(ROOT, PROFILE), encoding="utf-8").read()
    assert f"kernel_source_sha256_16: {hashlib.sha256(src).hexdigest()[:16]}" in text, \
        "the committed traffic summary was measured on other kernel sources"
    got = bench.measured_traffic()
    assert isinstance(got, int) and abs(got - 805306368) < 0.001 * 805306368  # the algorithmic bytes


def test_traffic_is_withheld_once_a_kernel_source_changes(tmp_path, monkeypatch):
    for f in HASHED:
        root = _tree(tmp_path / f, edit=f)
        monkeypatch.setattr(bench, "ROOT", str(root))
        assert bench.measured_traffic() is None


def test_traffic_is_withheld_without_the_summary(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    os.remove(root / PROFILE)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.measured_traffic() is None
