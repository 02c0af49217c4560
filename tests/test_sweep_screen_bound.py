"""The sweep's diagonal screen and its window sum bounds, checked on the CPU.

The sweep kernel skips the quadratic form e^T H e for a code when
mu2 * s > thr, with s = sum_i (e_i e_i) (H_ii / 2) in fp32, mu2 =
2 (1 - max_i r_i)(1 - 1e-4), r_i the Gershgorin row sums of H's
unit-diagonal scaling (screen on only for max r <= 0.9), and thr = best
(1 + 2e-5).  Its outputs equal the unscreened search's if every skipped
code's fp32 cost exceeds the best, which follows from two facts checked
here on H built to the limit (row sums up to 0.9, channel scales 1 to 40)
and on e chosen to make the bound tight:
  * e^T H e >= (1 - max r) sum_i H_ii e_i^2 (Gershgorin, exact arithmetic);
  * the fp32 form, in the kernel's order with fused multiply-adds, is within
    2e-5 relative of the exact form,
so mu2 * s stays below the fp32 cost times (1 + 2e-5).  fp32 fma is
emulated as one float64 multiply-add rounded to float32 (a product of two
floats is exact in float64)."""
import numpy as np


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _fma32(a, b, c):
    return _f32(a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64))


def _hessians(rng, n, rmax, tight=False):
    """n matrices D C D: C = I + A with A symmetric, |A| row sums <= rmax.
    tight: every off-diagonal entry of C is -rmax/15, so the smallest
    eigenvalue of C is exactly 1 - rmax (Gershgorin's bound is attained)."""
    if tight:
        a = np.broadcast_to(-(rmax / 15.0) * (np.ones((16, 16)) - np.eye(16)), (n, 16, 16))
    else:
        a = rng.uniform(0.0, 1.0, (n, 16, 16)) * rng.choice([-1.0, 1.0], (n, 16, 16))
        a = np.triu(a, 1)
        a = a + np.swapaxes(a, 1, 2)
        a *= (rmax / np.abs(a).sum(axis=2).max(axis=1))[:, None, None]
    c = np.eye(16) + a
    d = np.exp(rng.uniform(0.0, np.log(40.0), (n, 16)))
    return _f32(d[:, :, None] * c * d[:, None, :])


def _errors(rng, h):
    """Per H: random, mixed-magnitude and least-ratio error vectors (the
    minimiser of e^T H e / sum_i H_ii e_i^2, D^-1/2 times the least
    eigenvector of the unit-diagonal scaling), the last one perturbed."""
    n = h.shape[0]
    h64 = h.astype(np.float64)
    isd = 1.0 / np.sqrt(np.einsum("nii->ni", h64))
    _, vec = np.linalg.eigh(h64 * isd[:, :, None] * isd[:, None, :])
    least = vec[:, :, 0] * isd
    out = [rng.normal(0.0, 1.0, (n, 16)),
           rng.normal(0.0, 1.0, (n, 16)) * np.exp(rng.uniform(-8.0, 8.0, (n, 16))),
           least,
           least * (1.0 + 1e-3 * rng.normal(0.0, 1.0, (n, 16)))]
    return [_f32(e * rng.uniform(1e-3, 1e3, (n, 1))) for e in out]


def _screen_factor(h):
    h64 = h.astype(np.float64)
    dg = np.einsum("nii->ni", h64)
    r = (np.abs(h64) / np.sqrt(dg[:, :, None] * dg[:, None, :])).sum(axis=2) - 1.0
    rmax = r.max(axis=1)
    return rmax, np.where(rmax <= 0.9, _f32(2.0 * (1.0 - rmax) * (1.0 - 1e-4)), np.float32(0.0))


def _quad32(e, h):
    """2 * sum_i e_i (H_ii/2 e_i + sum_{j>i} H_ij e_j), the kernel's fp32 order."""
    hh = _f32(0.5 * np.einsum("nii->ni", h))
    acc = np.zeros(e.shape[0], np.float32)
    for i in range(16):
        v = _f32(hh[:, i].astype(np.float64) * e[:, i])
        for j in range(i + 1, 16):
            v = _fma32(h[:, i, j], e[:, j], v)
        acc = _fma32(e[:, i], v, acc)
    return _f32(2.0 * acc.astype(np.float64))


def _screen32(e, h):
    hh = _f32(0.5 * np.einsum("nii->ni", h))
    s = np.zeros(e.shape[0], np.float32)
    for i in range(16):
        s = _fma32(_f32(e[:, i].astype(np.float64) * e[:, i]), hh[:, i], s)
    return s


def test_screen_bound_and_rounding():
    rng = np.random.default_rng(11)
    for rlim, tight in [(r, t) for r in (0.0, 0.01, 0.3, 0.6, 0.9) for t in (False, True)]:
        h = _hessians(rng, 400, rlim * (1.0 - 1e-6), tight)   # fp32 rounding of H moves r by ~1e-7
        rmax, mu2 = _screen_factor(h)
        assert np.all(rmax <= 0.9) and np.all(mu2 > 0)
        h64 = h.astype(np.float64)
        for kind, e in enumerate(_errors(rng, h)):
            e64 = e.astype(np.float64)
            exact = np.einsum("ni,nij,nj->n", e64, np.triu(h64) + np.triu(h64, 1).swapaxes(1, 2), e64)
            diag = (np.einsum("nii->ni", h64) * e64 * e64).sum(axis=1)
            assert np.all(exact >= (1.0 - rmax) * diag * (1.0 - 1e-12))
            q32 = _quad32(e, h).astype(np.float64)
            assert np.all(np.abs(q32 - exact) <= 2e-5 * exact)
            bound = _f32(mu2.astype(np.float64) * _screen32(e, h)).astype(np.float64)
            assert np.all(bound < q32 * (1.0 + 2e-5))
            if tight and kind == 2:                    # the bound is attained up to its margin
                assert np.all(bound / q32 > 1.0 - 2e-4)


def test_screen_off_beyond_limit():
    rng = np.random.default_rng(12)
    for rlim in (0.95, 2.0):
        h = _hessians(rng, 50, rlim)
        rmax, mu2 = _screen_factor(h)
        assert np.all(mu2[rmax > 0.9] == 0)


def test_window_sum_bounds_are_lower_bounds():
    """The sweep closes a window side, where the screen is on, when
    (1 - max r) sum_i H_ii e_i^2 over the elements whose error is fixed
    beyond that side exceeds the threshold.  Checked on exact costs (the
    oracle's float64 cost of every code): for every code c,
      low:  (1 - max r) sum_i H_ii (|w_i| - 6 d_c)_+^2  <= min_{c' <= c} cost(c'),
      high: (1 - max r) sum_{|w_i| <= d_c / 4} H_ii w_i^2 <= min_{c' >= c} cost(c'),
    on H with row sums up to the screen's limit 0.9 (bound attained for the
    tight matrices), channel scales 1 to 40, and weights of mixed magnitude."""
    import datagen
    from oracle import nvfp4 as N
    from oracle import formats as F
    rng = np.random.default_rng(11)
    for rmax, tight in ((0.3, False), (0.9, False), (0.9, True)):
        h = _hessians(rng, 8, rmax, tight).astype(np.float64)            # 8 groups
        w = rng.laplace(0.0, 1.0, (64, 8 * 16)) * np.exp(rng.uniform(-3.0, 3.0, (64, 8 * 16)))
        bits = datagen.f32_to_bf16_bits(w.astype(np.float32))
        _, s2 = N.tensor_scale(bits)
        cost = N.sweep_costs(bits, h, s2)                                   # [64, 8, 127]
        wb = np.abs(F.bf16_bits_to_f64(bits)).reshape(64, 8, 16)
        hd = np.einsum("gii->gi", h)                                        # H_ii per group
        isd = 1.0 / np.sqrt(hd)
        r = (np.abs(h * isd[:, :, None] * isd[:, None, :]).sum(axis=2) - 1.0).max(axis=1)
        mu = 1.0 - r                                                        # per group
        d = N.block_scale(np.arange(127), s2)                               # [127]
        low_min = np.minimum.accumulate(cost, axis=2)                       # min over c' <= c
        high_min = np.minimum.accumulate(cost[:, :, ::-1], axis=2)[:, :, ::-1]
        for c in range(1, 127):
            el = np.maximum(wb - 6.0 * d[c], 0.0)
            lb_low = mu[None, :] * np.sum(hd[None, :, :] * el * el, axis=2)
            eh = np.where(wb <= d[c] / 4.0, wb, 0.0)
            lb_high = mu[None, :] * np.sum(hd[None, :, :] * eh * eh, axis=2)
            assert np.all(lb_low <= low_min[:, :, c] * (1 + 1e-12)), (rmax, c)
            assert np.all(lb_high <= high_min[:, :, c] * (1 + 1e-12)), (rmax, c)
