import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (run through the HIP library)")


# Parity tolerances (maximum relative error, row-normalised; see rel_err_rows).
TOL_F32 = 1e-3
TOL_BF16 = 2e-2


def rel_err_rows(got, ref):
    """Max over output rows of max_j |got_j - ref_j| / max_j |ref_j|.

    Output coordinates are convex combinations of N(0,1) values and can sit
    near zero, so the error of a row is measured against that row's largest
    magnitude.  A zero reference row (empty sequence) must be matched
    exactly (its denominator is replaced by 1).
    """
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    den = np.max(np.abs(ref), axis=1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.max(np.abs(got - ref), axis=1) / den))


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()
