"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_threads_do_not_change_results(orc):
    import numpy as np
    p = oracle_pins._rand_problem(21, batch=3, dim=5, L=77)
    y1, h1 = orc.scan(**p, nthreads=1)
    y4, h4 = orc.scan(**p, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(h1, h4)


def test_rows_subset_matches_full(orc):
    """Sampled rows (how full-size GPU runs are checked) give the same bits as
    the same rows inside a full call."""
    import numpy as np
    p = oracle_pins._rand_problem(22, batch=2, dim=4, L=50)
    y, h = orc.scan(**p)
    rb, rd = [1, 0, 1], [3, 2, 0]
    ys, hs = orc.scan_rows(p["x"][rb, rd], p["delta"][rb, rd], p["A"], p["B"], p["C"], rb, rd,
                           z_rows=p["z"][rb, rd], D=p["D"], delta_bias=p["delta_bias"])
    assert np.array_equal(ys, y[rb, rd]) and np.array_equal(hs, h[rb, rd])
