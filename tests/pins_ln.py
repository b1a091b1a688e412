"""Pins of the oracle's LayerNorm (forward and backward) against facts fixed outside it.

Each check takes an Oracle handle and raises AssertionError on a mismatch:
  * torch's float64 layer_norm and its autograd gradients on the CPU (a library
    routine computing the same real-number function; agreement to a few float64
    ulps, and the rounded outputs equal except where the two straddle a
    rounding midpoint);
  * exact values from Fraction/Decimal arithmetic on small rows;
  * exact invariances of the definition: negation, power-of-two scaling (eps = 0),
    constant rows, integer column sums for dbeta; identities of the gradient
    (its components along 1 and xhat vanish when eps = 0).
The definition pinned (Carbon README, "How It Works", LayerNorm row: float64
mean and variance): mean = sum(x)/H, var = sum((x-mean)^2)/H, rstd =
1/sqrt(var+eps), y = (x-mean)*rstd*gamma + beta, one rounding to the dtype.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import synthetic as syn
from tests.pins import stor, vals

DTS = ("f32", "bf16", "f16")


def _ulp_units(a, b, dt):
    """Distance in units of the last place between storage arrays a and b (same sign region)."""
    if dt == "f32":
        ia, ib = a.view(np.int32).astype(np.int64), b.view(np.int32).astype(np.int64)
    else:
        ia, ib = a.view(np.int16).astype(np.int64), b.view(np.int16).astype(np.int64)
    # map sign-magnitude codes onto a monotone integer line
    top = 1 << (31 if dt == "f32" else 15)
    ia = np.where(ia < 0, -(ia + top), ia)
    ib = np.where(ib < 0, -(ib + top), ib)
    return np.abs(ia - ib)


def _torch_fwd(dt, x, g, b, eps):
    import torch
    xt = torch.from_numpy(vals(x, dt))
    gt = torch.from_numpy(vals(g, dt)) if g is not None else None
    bt = torch.from_numpy(vals(b, dt)) if b is not None else None
    return torch.nn.functional.layer_norm(xt, (x.shape[1],), gt, bt, eps).numpy()


def _case(seed, dt, rows, h, scale=1.0, affine=True):
    x = syn.normal(seed, 0, (rows, h), sigma=scale, dt=dt)
    g = syn.normal(seed, 1, (h,), sigma=1.0, dt=dt) if affine else None
    b = syn.normal(seed, 2, (h,), sigma=0.5, dt=dt) if affine else None
    return x, g, b


def torch_forward(O):
    """Forward values within a few float64 ulps of torch's float64 layer_norm; rounded outputs equal
    except at a midpoint straddle (at most one unit apart, and rare)."""
    for dt in DTS:
        for si, (rows, h, scale, eps) in enumerate(((7, 100, 1.0, 1e-5), (5, 768, 3.0, 1e-5), (6, 33, 1e-3, 1e-5),
                                                    (4, 1, 1.0, 1e-5), (3, 257, 0.05, 1e-2))):
            x, g, b = _case(900 + si, dt, rows, h, scale)
            y, mean, rstd, r = O.layernorm_fwd(dt, x, g, b, eps=eps, want_r=True)
            t = _torch_fwd(dt, x, g, b, eps)
            xv = vals(x, dt)
            xhat = (xv - xv.mean(axis=1, keepdims=True)) / np.sqrt(xv.var(axis=1, keepdims=True) + eps)
            mag = np.abs(xhat * vals(g, dt)) + np.abs(vals(b, dt))
            assert np.all(np.abs(r - t) <= 64 * 2.0 ** -52 * mag), (dt, si, np.abs(r - t).max())
            yt = O.round_to(dt, t)   # the rounding itself is pinned by the downcast pins
            d = _ulp_units(y, yt, dt)
            assert d.max() <= 1 and (d > 0).mean() <= 0.01, (dt, si, int(d.max()), float((d > 0).mean()))
            assert np.all(np.abs(mean - xv.mean(axis=1)) <= 2.0 ** -45 * np.abs(xv).mean(axis=1)), (dt, si)
            assert np.allclose(rstd, 1.0 / np.sqrt(xv.var(axis=1) + eps), rtol=1e-12), (dt, si)


def decimal_forward(O):
    """Small rows against exact Fraction statistics and a 60-digit Decimal square root."""
    getcontext().prec = 60
    for dt in ("f32", "bf16"):
        for si, (h, eps) in enumerate(((40, 1e-5), (3, 0.25), (65, 0.0))):
            x, g, b = _case(950 + si, dt, 3, h)
            _, mean, rstd, r = O.layernorm_fwd(dt, x, g, b, eps=eps, want_r=True)
            xv, gv, bv = vals(x, dt), vals(g, dt), vals(b, dt)
            for i in range(3):
                mu = sum((Fraction(v) for v in xv[i]), Fraction(0)) / h
                var = sum(((Fraction(v) - mu) ** 2 for v in xv[i]), Fraction(0)) / h
                den = (Decimal(var.numerator) / Decimal(var.denominator) + Decimal(eps)).sqrt()
                assert abs(Fraction(mean[i]) - mu) <= Fraction(2.0 ** -50) * abs(mu) + Fraction(2.0 ** -1000)
                rs = Decimal(1) / den
                assert abs(Decimal(rstd[i]) - rs) <= Decimal(2.0 ** -49) * rs, (dt, si, i)
                for j in range(h):
                    ex = (Decimal(xv[i, j]) - Decimal(mu.numerator) / Decimal(mu.denominator)) * rs * Decimal(gv[j]) \
                        + Decimal(bv[j])
                    tol = Decimal(2.0 ** -46) * (abs(Decimal(gv[j])) * (abs(Decimal(xv[i, j]) * rs) + 1) + abs(Decimal(bv[j])))
                    assert abs(Decimal(r[i, j]) - ex) <= tol, (dt, si, i, j, r[i, j], ex)


def invariances(O):
    """Negation (no beta), power-of-two scaling (eps = 0) and constant rows, all bit for bit."""
    for dt in DTS:
        x, g, b = _case(970, dt, 6, 130)
        y, mean, rstd, _ = O.layernorm_fwd(dt, x, g, None)
        xn = stor(-vals(x, dt), dt)
        yn, mn, rn, _ = O.layernorm_fwd(dt, xn, g, None)
        assert np.array_equal(stor(-vals(y, dt), dt), yn) and np.array_equal(mn, -mean) and np.array_equal(rn, rstd), dt
        y0, m0, r0, _ = O.layernorm_fwd(dt, x, g, b, eps=0.0)
        for k in (-3, 2):
            xs = stor(vals(x, dt) * 2.0 ** k, dt)
            assert np.array_equal(vals(xs, dt), vals(x, dt) * 2.0 ** k)
            ys, ms, rs, _ = O.layernorm_fwd(dt, xs, g, b, eps=0.0)
            assert np.array_equal(ys, y0), (dt, k)
            assert np.array_equal(ms, m0 * 2.0 ** k) and np.array_equal(rs, r0 * 2.0 ** -k), (dt, k)
        c = stor(np.full((3, 77), 1.5) * np.array([[1.0], [-3.0], [0.0]]), dt)
        yc, mc, rc, _ = O.layernorm_fwd(dt, c, g[:77], b[:77])
        assert np.array_equal(yc, np.stack([b[:77]] * 3)), dt
        assert np.array_equal(mc, np.array([1.5, -4.5, 0.0])) and np.all(rc == 1.0 / np.sqrt(1e-5)), dt
        # no affine: the normalised row itself; a two-valued row normalises to +-1 (up to eps)
        yv, _, _, rv = O.layernorm_fwd(dt, stor(np.array([[2.0, -2.0] * 8]), dt), None, None, eps=0.0, want_r=True)
        assert np.array_equal(rv, np.array([[1.0, -1.0] * 8])), dt


def _torch_bwd(dt, dy, x, g, eps):
    import torch
    xt = torch.from_numpy(vals(x, dt)).requires_grad_(True)
    gt = torch.from_numpy(vals(g, dt)).requires_grad_(True) if g is not None else None
    bt = torch.zeros(x.shape[1], dtype=torch.float64, requires_grad=True)
    out = torch.nn.functional.layer_norm(xt, (x.shape[1],), gt, bt, eps)
    out.backward(torch.from_numpy(vals(dy, dt)))
    return xt.grad.numpy(), (gt.grad.numpy() if gt is not None else None), bt.grad.numpy()


def torch_backward(O):
    """dx, dgamma, dbeta within float64 rounding of torch's autograd (float64, CPU)."""
    for dt in DTS:
        for si, (rows, h, eps, affine) in enumerate(((9, 100, 1e-5, True), (70, 48, 1e-5, True), (5, 257, 0.1, False),
                                                     (33, 1, 1e-5, True))):
            x, g, _ = _case(1000 + si, dt, rows, h, 2.0, affine)
            dy = syn.normal(1000 + si, 3, (rows, h), dt=dt)
            _, mean, rstd, _ = O.layernorm_fwd(dt, x, g, None, eps=eps)
            dx, dg, dbt, rdx = O.layernorm_bwd(dt, dy, x, mean, rstd, g, pdt="f32", want_r=True)
            tx, tg, tb = _torch_bwd(dt, dy, x, g, eps)
            sc = np.abs(vals(dy, dt)).max() * (np.abs(vals(g, dt)).max() if affine else 1.0) * rstd.max()
            assert np.abs(rdx - tx).max() <= 2.0 ** -40 * sc * h, (dt, si, np.abs(rdx - tx).max())
            assert np.abs(dg.astype(np.float64) - tg).max() <= 2.0 ** -22 * (np.abs(tg).max() + 1) if affine else True
            assert np.abs(dbt.astype(np.float64) - tb).max() <= 2.0 ** -22 * (np.abs(tb).max() + 1), (dt, si)
            if h == 1:   # the normalised value is identically 0, so is its gradient
                assert np.all(rdx == 0.0), (dt, si)
                continue
            d = _ulp_units(dx, O.round_to(dt, tx), dt)
            assert d.max() <= 1 and (d > 0).mean() <= 0.02, (dt, si, int(d.max()))


def gradient_identities(O):
    """With eps = 0 the gradient is orthogonal to 1 and to xhat (the forward ignores shifts and scales)."""
    for dt in ("f32", "bf16"):
        x, g, _ = _case(1050, dt, 8, 96, 1.0)
        dy = syn.normal(1050, 3, (8, 96), dt=dt)
        _, mean, rstd, _ = O.layernorm_fwd(dt, x, g, None, eps=0.0)
        _, _, _, rdx = O.layernorm_bwd(dt, dy, x, mean, rstd, g, want_r=True)
        xhat = (vals(x, dt) - mean[:, None]) * rstd[:, None]
        mag = (np.abs(rdx) * (1 + np.abs(xhat))).sum(axis=1)
        assert np.all(np.abs(rdx.sum(axis=1)) <= 2.0 ** -45 * mag), dt
        assert np.all(np.abs((rdx * xhat).sum(axis=1)) <= 2.0 ** -45 * mag), dt


def dbeta_integer_exact(O):
    """dbeta is the exact column sum for integer dY; dgamma likewise when xhat is exact (x = +-1 rows)."""
    for dt in DTS:
        rows, h = 130, 20
        dy = syn.integers(1060, 3, (rows, h), -8, 8, dt)
        x = stor(np.where(syn.integers(1060, 0, (rows, h), 0, 2, "f32") > 0, 1.0, -1.0) * np.ones((rows, h)), dt)
        x[:, 0] = stor(np.ones(rows), dt)
        x[:, 1] = stor(-np.ones(rows), dt)
        _, mean, rstd, _ = O.layernorm_fwd(dt, x, None, None, eps=0.0)
        _, dg, dbt, _ = O.layernorm_bwd(dt, dy, x, mean, rstd, None, pdt="f32")
        assert np.array_equal(dbt.astype(np.float64), vals(dy, dt).sum(axis=0)), dt
        xhat = (vals(x, dt) - mean[:, None]) * rstd[:, None]
        dyv = vals(dy, dt)
        ex = [sum((Fraction(a) * Fraction(b) for a, b in zip(dyv[:, j], xhat[:, j])), Fraction(0)) for j in range(h)]
        mag = np.abs(dyv * xhat).sum(axis=0)
        assert all(abs(Fraction(float(v)) - e) <= Fraction(2.0 ** -23) * abs(e) + Fraction(2.0 ** -40 * float(mg))
                   for v, e, mg in zip(dg.astype(np.float64), ex, mag)), dt


ALL = [torch_forward, decimal_forward, invariances, torch_backward, gradient_identities, dbeta_integer_exact]
