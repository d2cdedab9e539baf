"""bench.py contract on the host: the one-GPU refusal and the algorithmic byte model.

The byte model counts what the method moves per point: the point (4 d bytes), the
encoder's output rows, one 4-byte read per table value a point references (2^d corners of
F features per level for the d-linear interpolant; 2^d corners times 2^d coefficients for
the Hermite one) and, in the backward, one 8-byte read-modify-write per scattered value.
The expected figures below are worked out by hand from those counts.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (imports no GPU module at load time)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_bytes_per_point_dlinear_3d_l16():
    # forward: 12 (x) + 16 levels x 2 features x 4 B (row) + 16 x 8 corners x 2 x 4 B = 1164
    # backward: 12 + 128 (upstream row) + 16 x 8 x 2 x 8 B (atomic read-modify-write) = 2188
    spec = {"d": 3, "L": 16, "F": 2, "kind": "dlinear"}
    assert bench.algorithmic_bytes_per_point(spec) == {"forward": 1164, "backward": 2188}


def test_bytes_per_point_dlinear_active_levels():
    # 8 of 16 levels active: the forward still writes the full 16-level row (128 B), while
    # gathers (8 x 8 x 2 x 4 = 512), upstream (8 x 2 x 4 = 64) and scatters (8 x 8 x 2 x 8 =
    # 1024) cover the active levels only
    spec = {"d": 3, "L": 16, "F": 2, "kind": "dlinear", "active_levels": 8}
    assert bench.algorithmic_bytes_per_point(spec) == {"forward": 12 + 128 + 512, "backward": 12 + 64 + 1024}


@pytest.mark.parametrize("d2_mode,comps", [("diag", 7), ("laplacian", 5)])
def test_bytes_per_point_hermite_3d(d2_mode, comps):
    # outputs per level: value, 3 gradient components and 3 diagonal second derivatives (or
    # one Laplacian); 8 corners x 8 coefficients (all mixed partials) of 2 features each
    spec = {"d": 3, "L": 16, "F": 2, "kind": "hermite", "d2_mode": d2_mode}
    rows = 4 * 16 * 2 * comps
    assert bench.algorithmic_bytes_per_point(spec) == {
        "forward": 12 + rows + 4 * 16 * 64 * 2,
        "backward": 12 + rows + 8 * 16 * 64 * 2,
    }
