"""The oracle's process pool (tests/_pool.py) returns what the oracle returns
when called directly, piece by piece and stitched together (small inputs)."""
import numpy as np
import pytest

import datagen
from oracle import nvfp4 as N
from oracle import mxcast as M

import _pool


@pytest.fixture(scope="module")
def pool():
    p = _pool.make_pool()
    yield p
    p.shutdown()


def test_pool_sweep_costs_match(pool):
    w, x = datagen.config1()
    h = N.hessian(x)
    s2 = N.tensor_scale(w)[1]
    got = _pool.sweep_costs(pool, w, h, s2, rows_per_item=7)
    ref = N.sweep_costs(w, h, s2)
    # float64 sums in another blocking order: equal to rounding, same argmin
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    assert np.array_equal(np.argmin(got, axis=2), np.argmin(ref, axis=2))


def test_pool_hessian_pieces_add_up(pool):
    _, x = datagen.config1()
    futs = [(c0, pool.submit(_pool.hessian_piece, np.ascontiguousarray(x[t0:t0 + 128, c0:c0 + 64])))
            for c0 in range(0, 256, 64) for t0 in range(0, 512, 128)]
    h = np.zeros((16, 16, 16))
    amax = 0.0
    for c0, f in futs:
        hp, a = f.result()
        h[c0 // 16:c0 // 16 + 4] += hp
        amax = max(amax, a)
    ref = N.hessian(x)
    assert np.allclose(h, ref, rtol=1e-12, atol=0)
    assert amax == N.tensor_scale(x)[0]


def test_pool_cast_matches(pool):
    p, e, _ = datagen.config5(experts=3, rows=16, k=256, forced_frac=0.05)
    got = _pool.cast(pool, p, e)
    ref = M.mxfp4_to_nvfp4(p, e)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
