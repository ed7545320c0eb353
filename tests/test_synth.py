"""The seeded workload generator: deterministic, right shapes and outlier structure."""
import numpy as np

from synth import CONFIGS, alpha_grid, make_layer, row_subset, small_spec


def test_c1_deterministic_and_shaped():
    a = make_layer(CONFIGS["c1"][0])
    b = make_layer(CONFIGS["c1"][0])
    assert a.W.dtype == np.float16 and a.X.dtype == np.float16
    assert a.W.shape == (512, 512) and a.X.shape == (256, 512)
    assert np.array_equal(a.W, b.W) and np.array_equal(a.X, b.X)
    assert len(a.outlier_channels) == 5 and np.all(a.outlier_factors == 20.0)
    col = np.abs(a.X.astype(np.float64)).mean(axis=0)
    others = np.delete(col, a.outlier_channels)
    assert col[a.outlier_channels].min() > 8 * others.max()
    assert 0.015 < a.W.astype(np.float64).std() < 0.025


def test_config_table():
    shapes = {s.name: (s.out_features, s.in_features, s.n_tokens, s.w_bit, s.group_size,
                       s.zero_point, s.outlier_count)
              for specs in CONFIGS.values() for s in specs}
    assert shapes["c1"] == (512, 512, 256, 4, 128, 0, 5)
    assert shapes["c2"] == (4096, 4096, 4096, 4, 128, 1, 41)
    assert shapes["c3_up"] == (11008, 4096, 16384, 4, 128, 1, 41)
    assert shapes["c3_down"] == (4096, 11008, 16384, 4, 128, 1, 110)
    assert shapes["c4"] == (28672, 8192, 65536, 4, 128, 1, 41)
    assert shapes["c5"] == (13824, 5120, 32768, 3, 64, 1, 51)


def test_loguniform_factors_and_t4():
    spec = small_spec("t", 64, 256, 300, x_dist="t4", outlier_count=9,
                      outlier_factor=("loguniform", 10.0, 50.0))
    L = make_layer(spec)
    assert np.all((L.outlier_factors >= 10.0) & (L.outlier_factors <= 50.0))
    assert L.X.shape == (300, 256)


def test_row_subset_and_alpha_grid():
    s = CONFIGS["c4"][0]
    r = row_subset(s, 512)
    assert len(r) == 512 and np.all(np.diff(r) > 0) and r.max() < s.out_features
    assert np.array_equal(r, row_subset(s, 512))
    g = alpha_grid(20)
    assert g.dtype == np.float32 and g[0] == 0 and g[-1] == 1 and len(g) == 20
