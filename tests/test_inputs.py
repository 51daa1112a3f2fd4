"""The seeded generators: determinism, CSR well-formedness, family shapes."""
import numpy as np
import pytest

import mce_inputs as mi
import oracle


def well_formed(g):
    assert g.row_ptr.dtype == np.int32 and g.col_idx.dtype == np.int32
    assert g.row_ptr.shape == (g.n + 1,) and g.row_ptr[0] == 0 and g.row_ptr[-1] == g.nnz
    assert oracle.validate(g.n, g.row_ptr, g.col_idx) == 0


@pytest.mark.parametrize("make", [
    lambda s: mi.erdos_renyi(300, 0.05, s),
    lambda s: mi.rmat(10, 8, 0.57, 0.19, 0.19, 0.05, s),
    lambda s: mi.chung_lu(3000, 10.0, 2.3, None, s, planted=5),
    lambda s: mi.random_small(20, 0.4, s),
])
def test_seeded_and_well_formed(make):
    a, b, c = make(3), make(3), make(4)
    well_formed(a)
    assert a.sha256() == b.sha256()
    assert a.sha256() != c.sha256()


def test_from_edges_cleans_input():
    g = mi.from_edges(4, [0, 1, 1, 2, 3, 3], [1, 0, 1, 3, 2, 2])
    assert g.edge_list().tolist() == [[0, 1], [2, 3]]
    well_formed(g)


def test_config_small_shapes():
    g0 = mi.config_graph(0)
    well_formed(g0)
    assert g0.n == 2000 and abs(g0.m - 0.01 * 2000 * 1999 / 2) < 800
    g1 = mi.config_graph(1)
    well_formed(g1)
    assert g1.n == 45 and g1.m == 945 and set(g1.degrees().tolist()) == {42}


def test_chung_lu_weights_hit_targets():
    w = mi._chung_lu_weights(500_000, 30.0, 2.3, 3872.98)
    assert abs(w.mean() - 30.0) < 1e-6 * 30 and abs(w[0] - 3872.98) < 1e-6 * 3872.98
    assert np.all(np.diff(w) < 0)


def test_erdos_renyi_degree_mean():
    g = mi.erdos_renyi(1500, 0.02, 11)
    assert abs(g.degrees().mean() - 0.02 * 1499) < 1.0
