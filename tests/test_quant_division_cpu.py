"""The quantiser kernel rounds w / scale to an integer without dividing:
it takes p = fl(w * fl(1 / scale)) and divides only where p lies within
2^-14 of a half-integer.  This checks that rule in binary32 on the CPU, on
quotients packed around every half-integer of the int8 range, against the
plain rint(fl(w / scale)) the pages' rounding step asks for."""
import numpy as np

F = np.float32


def _near_half_inputs(rng, n_scales=40, ulps=6):
    ws, ss = [], []
    for s in rng.uniform(1e-6, 1.0, n_scales).astype(F):
        c = F(s) * F(127.0)
        scale = F(c / F(127.0))
        h = (np.arange(-128, 128) + 0.5).astype(F)
        centre = (h * scale).astype(F)
        for k in range(-ulps, ulps + 1):
            v = centre
            step = np.inf if k > 0 else -np.inf
            for _ in range(abs(k)):
                v = np.nextafter(v, F(step)).astype(F)
            v = np.clip(v, -c, c).astype(F)
            ws.append(v)
            ss.append(np.full(v.shape, scale, F))
    return np.concatenate(ws), np.concatenate(ss)


def test_multiply_then_divide_near_half_integers_matches_division():
    rng = np.random.default_rng(11)
    w, scale = _near_half_inputs(rng)
    exact = np.rint(w / scale)
    inv = (F(1.0) / scale).astype(F)   # the kernel uses v_rcp_f32 (1 ulp); the bound covers both
    p = (w * inv).astype(F)
    near = np.abs(p - np.floor(p) - F(0.5)) < F(2.0 ** -14)
    r = np.where(near, w / scale, p).astype(F)
    assert np.array_equal(np.rint(r), exact)
    # the inputs do reach the exact ties and the cases where p alone rounds
    # the other way, so the division branch is exercised
    q = (w / scale).astype(F)
    assert np.any(q - np.floor(q) == F(0.5))
    assert np.any(np.rint(p) != exact)
    assert near.any() and not near.all()


def test_multiply_rule_on_ordinary_rows():
    rng = np.random.default_rng(12)
    for _ in range(20):
        w = rng.normal(0, 0.02, 4096).astype(F)
        c = np.abs(w).max().astype(F)
        scale = F(c / F(127.0))
        exact = np.rint(w / scale)
        p = (w * (F(1.0) / scale)).astype(F)
        near = np.abs(p - np.floor(p) - F(0.5)) < F(2.0 ** -14)
        assert np.array_equal(np.rint(np.where(near, w / scale, p)), exact)
