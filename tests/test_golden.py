"""Pins of the oracle to values the pages print (fixtures under tests/golden/, each citing
its page and section)."""
import os

import numpy as np
import pytest

from multiresolution_hash_grid_multires_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _basis_fixture():
    coef, rows = {}, []
    for line in open(os.path.join(GOLDEN, "hermite_basis_far_corner.txt")):
        f = line.split("#")[0].split()
        if not f:
            continue
        if f[0] == "coef":
            coef[f[1]] = [float(v) for v in f[2:]]
        elif f[0] == "value":
            rows.append([float(v) for v in f[1:]])
    return coef, np.array(rows)


def test_fixture_values_match_printed_polynomials():
    coef, rows = _basis_fixture()
    for j, name in enumerate(("h0", "h1", "dh0", "d2h0")):
        np.testing.assert_array_equal(np.polynomial.polynomial.polyval(rows[:, 0], coef[name]), rows[:, 1 + j])


@pytest.mark.parametrize("N", [4, 8])
def test_oracle_reproduces_printed_far_corner_bases(orc, N):
    # One dense 2D level of resolution N; a single non-zero coefficient at vertex (1, 0):
    # the value slot gives gamma = h0(t), d/dx = N h0'(t), d2/dx2 = N^2 h0''(t) along the
    # x edge (t1 = 0); the x-derivative slot gives gamma = (1/N) h1(t).
    _, rows = _basis_fixture()
    t = rows[:, 0]
    spec = {"d": 2, "L": 1, "F": 1, "kind": "hermite", "T": [1 << 12] * 3, "n_min": N, "n_max": N,
            "d2_mode": "diag"}
    lay = orc.layout(spec)
    x = np.stack([t / N, np.zeros_like(t)], axis=1).astype(np.float32)
    row = 1  # vertex (1, 0), x fastest
    for table, slot, expect_g, scale in ((0, 0, rows[:, 1], 1.0), (1, 0, rows[:, 2], 1.0 / N)):
        params = np.zeros(lay["n_params"])
        params[lay["offset"][table, 0] + row * lay["width"][table, 0] + slot] = 1.0
        g, dg, d2 = orc.forward(spec, x, params)
        np.testing.assert_allclose(g[:, 0], scale * expect_g, rtol=0, atol=1e-15)
        if table == 0:
            np.testing.assert_allclose(dg[:, 0, 0], N * rows[:, 3], rtol=0, atol=1e-12)
            np.testing.assert_allclose(d2[:, 0, 0], N * N * rows[:, 4], rtol=0, atol=1e-9)


def test_workloads_follow_the_page_configurations():
    facts = {}
    for line in open(os.path.join(GOLDEN, "page_configs.txt")):
        f = line.split("#")[0].split("=")
        if len(f) == 2:
            facts[f[0].strip()] = int(f[1])
    s = I.WORKLOADS["dlinear3d_L16_T19"]["spec"]
    assert (s["L"], s["F"], s["T"][0]) == (facts["ingp_levels"], facts["ingp_features"], 1 << facts["ingp_table_log2"])
    assert I.WORKLOADS["hermite2d_L8_T14"]["spec"]["T"][0] == 1 << facts["hermite_table_log2"]
    assert I.WORKLOADS["pinn_residual3d"]["mlp"]["omega"] == facts["siren_omega0"]
    assert I.WORKLOADS["hermite2d_L8_T14_14_10"]["spec"]["T"] == [1 << facts[f"hermite_best_t{k}_log2"] for k in range(3)]
