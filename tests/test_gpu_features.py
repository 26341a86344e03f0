"""The gfx950 lane layouts the kernel relies on (transposing LDS read,
half-wave swap, direct-to-LDS buffer loads with zero fill), checked on the
GPU by the calibration tool's --check mode."""
import os
import subprocess

import pytest

from exact_io_aware_25_amd import _build

pytestmark = pytest.mark.gpu


def test_lane_layouts_hold():
    assert os.path.exists(_build.CALIBRATE), "build first"
    print("[gpu-case] calibrate_gfx950 --check", flush=True)
    r = subprocess.run([_build.CALIBRATE, "--check"], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
