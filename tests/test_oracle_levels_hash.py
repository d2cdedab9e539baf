"""Oracle pins: level progression, spatial hash, dense 1:1 indexing, position stage.

Sources: Instant-NGP explainer (nxrte.com), "InstantNGP 与多分辨率哈希编码流程与原理"
(the 2^d vertices per level, the spatial hash spreading neighbours randomly over the
table, the 1:1 map at coarse levels); Instant-NGP news article (antipu.com.cn),
adaptivity paragraph (1:1 at low resolution, hashed at high) and the Figure 3 paragraph
(levels in geometric progression between N_min and N_max).
"""
import math

import numpy as np
import pytest

P1, P2 = 2654435761, 805459861


# ---------------------------------------------------------------- levels
def test_levels_exact_geometric_series(orc):
    # growth 1.5 from 16: every N_min * b^l is an integer, so the series is exact.
    assert orc.levels(4, 16, 0, 1.5) == [16, 24, 36, 54]
    assert orc.levels(5, 3, 0, 2.0) == [3, 6, 12, 24, 48]


@pytest.mark.parametrize("L,nmin,nmax", [(8, 16, 512), (16, 16, 2048), (16, 16, 1024), (12, 4, 4096)])
def test_levels_endpoints_and_progression(orc, L, nmin, nmax):
    N = orc.levels(L, nmin, nmax)
    assert N[0] == nmin and N[-1] == nmax          # both ends of [N_min, N_max]
    b = math.exp((math.log(nmax) - math.log(nmin)) / (L - 1))
    for l, n in enumerate(N):
        exact = nmin * b ** l
        assert exact - 1 + 1e-9 < n <= exact + 1e-6 + 1e-9   # the floor of the geometric term
    assert all(a < c for a, c in zip(N, N[1:]))


def test_levels_power_of_two_endpoints_not_lost(orc):
    # 16 * 2^(6 l / 15) hits 64, 256, 1024 exactly; fp64 pow lands just below for some l.
    N = orc.levels(16, 16, 1024)
    assert N[5] == 64 and N[10] == 256 and N[15] == 1024


# ---------------------------------------------------------------- hash
def test_hash_x_axis_is_identity(orc):
    # the first prime is 1: vertices on the x axis hash to themselves
    for v in [0, 1, 81, 12345, 2 ** 31 + 7]:
        assert orc.hash_vertex([v, 0, 0]) == v
        assert orc.hash_vertex([v, 0]) == v


def test_hash_unit_vertices_give_the_primes(orc):
    assert orc.hash_vertex([0, 1, 0]) == P1
    assert orc.hash_vertex([0, 0, 1]) == P2
    assert orc.hash_vertex([0, 1]) == P1
    # the fourth (time) axis of the space-time grid takes the next prime of the same list
    assert orc.hash_vertex([0, 0, 0, 1]) == 3674653429
    v = [5, 7, 11, 13]
    M = 1 << 32
    assert orc.hash_vertex(v) == 5 ^ (7 * P1 % M) ^ (11 * P2 % M) ^ (13 * 3674653429 % M)
    assert orc.hash_vertex(v) == orc.hash_vertex([5, 7, 11, 0]) ^ orc.hash_vertex([0, 0, 0, 13])


def test_hash_combines_axes_by_xor(orc):
    rng = np.random.default_rng(0)
    for _ in range(200):
        v = [int(a) for a in rng.integers(0, 1 << 20, size=3)]
        h = orc.hash_vertex(v)
        parts = orc.hash_vertex([v[0], 0, 0]) ^ orc.hash_vertex([0, v[1], 0]) ^ orc.hash_vertex([0, 0, v[2]])
        assert h == parts
        # an additive combination would differ for most vertices; XOR is self-inverse
        assert h ^ orc.hash_vertex([0, v[1], 0]) == orc.hash_vertex([v[0], 0, v[2]])


def test_hash_products_wrap_mod_2_32(orc):
    # 2 * 2654435761 = 5308871522 exceeds 2^32; the product wraps to 1013904226
    assert orc.hash_vertex([0, 2, 0]) == 1013904226
    assert orc.hash_vertex([0, 0, 8]) == (8 * P2) % (1 << 32)


def test_hashed_level_index_is_hash_mod_T_nonpow2(orc):
    # a T that is not a power of two: the index is the uint32 hash reduced mod T
    spec = {"d": 2, "L": 1, "F": 1, "kind": "dlinear", "T": [1000], "resolutions": [100]}
    x = np.array([[0.0, 2.0 / 100 + 1e-4]], np.float32)  # base (0, 2)
    idx = orc.indices(spec, x)[0, 0]
    assert idx[0] == 1013904226 % 1000 == 226
    assert idx[1] == (1 ^ 1013904226) % 1000


def test_hash_spreads_rows_uniformly(orc):
    # vertices of random cells of a fine level land evenly over the table
    spec = {"d": 3, "L": 1, "F": 1, "kind": "dlinear", "T": [1 << 12], "resolutions": [255]}
    x = np.random.default_rng(1).random((1 << 18, 3), dtype=np.float32)
    idx = orc.indices(spec, x)[:, 0, 0]
    counts = np.bincount(idx, minlength=1 << 12)
    expected = idx.size / (1 << 12)
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    dof = (1 << 12) - 1
    assert abs(chi2 - dof) < 6 * math.sqrt(2 * dof)
    assert idx.max() < (1 << 12) and idx.min() >= 0


def test_hash_covers_the_table(orc):
    # every row of a hashed level is reachable: the 64^3 vertices of a level cover 2^12 rows
    spec = {"d": 3, "L": 1, "F": 1, "kind": "dlinear", "T": [1 << 12], "resolutions": [63]}
    g = (np.arange(63) + 0.5) / 63
    x = np.stack(np.meshgrid(g, g, g, indexing="ij"), -1).reshape(-1, 3).astype(np.float32)
    idx = orc.indices(spec, x)[:, 0, :]
    assert np.unique(idx).size == 1 << 12


# ---------------------------------------------------------------- dense levels
@pytest.mark.parametrize("d,N", [(2, 16), (2, 54), (3, 16), (3, 30), (4, 6)])
def test_dense_level_is_a_bijection_x_fastest(orc, d, N):
    spec = {"d": d, "L": 1, "F": 1, "kind": "dlinear", "T": [1 << 19], "resolutions": [N]}
    lay = orc.layout(spec)
    assert lay["dense"][0, 0] and lay["rows"][0, 0] == (N + 1) ** d
    c = (np.arange(N) + 0.5) / N
    x = np.stack(np.meshgrid(*([c] * d), indexing="ij"), -1).reshape(-1, d).astype(np.float32)
    idx = orc.indices(spec, x)[:, 0, :]
    seen = np.unique(idx)
    assert seen.size == (N + 1) ** d and seen[0] == 0 and seen[-1] == (N + 1) ** d - 1
    # corner 0 of cell (i, j, k) is row i + j (N+1) + k (N+1)^2; corner bit 0 moves +1 in x
    base = np.floor(x.astype(np.float64) * N).astype(np.int64)
    expect0 = sum(base[:, i] * (N + 1) ** i for i in range(d))
    assert np.array_equal(idx[:, 0], expect0)
    for i in range(d):
        assert np.array_equal(idx[:, 1 << i], expect0 + (N + 1) ** i)


def test_dense_switch_follows_vertex_count(orc):
    # (N+1)^d <= T is dense; one more vertex than rows is hashed
    spec = {"d": 2, "L": 2, "F": 1, "kind": "dlinear", "T": [64 * 64], "resolutions": [63, 64]}
    lay = orc.layout(spec)
    assert lay["dense"][0].tolist() == [True, False]
    assert lay["rows"][0].tolist() == [64 * 64, 64 * 64]


def test_hermite_tables_decide_density_per_table(orc):
    # per-order table sizes can differ; each table decides 1:1 vs hash on its own size
    spec = {"d": 2, "L": 2, "F": 2, "kind": "hermite", "T": [1 << 10, 1 << 6, 1 << 10],
            "resolutions": [7, 31]}
    lay = orc.layout(spec)
    assert lay["dense"].tolist() == [[True, True], [True, False], [True, True]]
    assert lay["width"][:, 0].tolist() == [2, 4, 2]
    assert lay["rows"].tolist() == [[64, 1024], [64, 64], [64, 1024]]
    off = lay["offset"].ravel()
    sizes = (lay["rows"] * lay["width"]).ravel()
    assert np.array_equal(off[1:], np.cumsum(sizes)[:-1]) and off[0] == 0
    assert lay["n_params"] == sizes.sum()


# ---------------------------------------------------------------- position stage
def test_position_edges(orc):
    spec = {"d": 1, "L": 1, "F": 1, "kind": "dlinear", "T": [1 << 10], "resolutions": [16]}
    x = np.array([[0.0], [1.0], [0.25], [np.nextafter(np.float32(0.25), np.float32(0))],
                  [-0.5], [1.5]], np.float32)
    idx = orc.indices(spec, x)[:, 0, :]
    assert idx[0].tolist() == [0, 1]        # x = 0: first cell
    assert idx[1].tolist() == [15, 16]      # x = 1: last cell (t = 1), never past the grid
    assert idx[2].tolist() == [4, 5]        # exactly on a vertex: the upper cell, t = 0
    assert idx[3].tolist() == [3, 4]        # just below a vertex: the lower cell
    assert idx[4].tolist() == [0, 1]        # clamped below
    assert idx[5].tolist() == [15, 16]      # clamped above


def test_position_uses_one_rounded_fp32_product(orc):
    # x * N rounded once in fp32 decides the cell; with N = 3 many x land exactly on a
    # vertex only after rounding
    spec = {"d": 1, "L": 1, "F": 1, "kind": "dlinear", "T": [1 << 10], "resolutions": [3]}
    x = np.float32(1.0) / np.float32(3.0)  # fl(1/3) * 3 rounds to exactly 1
    assert np.float32(x) * np.float32(3.0) == np.float32(1.0)
    idx = orc.indices(spec, np.array([[x]], np.float32))[0, 0]
    assert idx.tolist() == [1, 2]
