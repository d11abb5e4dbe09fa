"""The approximation study runs on the CPU and its numbers are sane."""
import numpy as np

from oracle import approx_study


def test_study_small():
    rows = dict((n, (d, i)) for n, d, i in approx_study.study(T=64, dk=8, dv=4, heads=2))
    assert set(rows) == set(approx_study.REGIMES)
    for n, (d, i) in rows.items():
        assert np.isfinite(d) and np.isfinite(i) and 0 <= d < 10 and 0 < i < 10, n
    # axis-aligned keys keep the covariance diagonal: the diagonal filter is exact
    assert rows["axis keys"][0] < 1e-10
    # with generic keys the mean-field diagonal filter tracks the exact one
    # more closely than the single-scalar isotropic filter
    assert rows["random keys"][0] < rows["random keys"][1]
