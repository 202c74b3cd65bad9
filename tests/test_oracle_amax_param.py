"""Pins of the amax reparameterization of scale learning ("Scale Learning:
Training NVFP4 Block Scales", How Scale Learning Works: the trained quantity
is the block amax, s = amax / 6): the forward reduces to the scale form, the
gradients are the scale gradients times ds/da = 1/6, finite differences in
the post amax, and the tied identity.  CPU only."""
import numpy as np

import oracle as O


def _case(rows=8, cols=64, seed=0, dual=False, exact=False):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    u = x.view(np.uint32)
    x = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).view(np.float32)  # bf16 values
    g = (rng.standard_normal((rows, cols)) * 1e-3).astype(np.float32)
    nb = rows * cols // 16
    if exact:
        # s with few significant bits, a = 6 s exactly: a / 6 and q * s are exact
        s = (2.0 ** rng.integers(-12, -6, nb) * rng.choice([1.0, 1.25, 1.5, 1.75], nb)).astype(np.float32)
        a = (6.0 * s).astype(np.float32)
    else:
        a = (np.abs(x).reshape(-1, 16).max(axis=1) * rng.uniform(0.7, 1.3, nb)).astype(np.float32)
    a = a.reshape(rows, cols // 16)
    ap = None
    if dual:
        ap = (a * np.float32(1.125)).astype(np.float32)
    return x, g, a, ap


def test_forward_is_the_scale_form_at_a_over_6():
    for dual in (False, True):
        x, g, a, ap = _case(dual=dual, seed=1)
        s = (a / np.float32(6)).astype(np.float32)
        sp = None if ap is None else (ap / np.float32(6)).astype(np.float32)
        assert np.array_equal(O.fakequant_fwd(x, a, ap, amax=True), O.fakequant_fwd(x, s, sp))


def test_gradients_are_the_scale_gradients_over_6():
    x, g, a, _ = _case(seed=2, rows=32)
    s = (a / np.float32(6)).astype(np.float32)
    dx_a, da = O.fakequant_bwd(x, g, a, amax=True)
    dx_s, ds = O.fakequant_bwd(x, g, s)
    assert np.array_equal(dx_a, dx_s)
    # both are the same binary64 block sum, rounded once: ds = fl(S), da = fl(S / 6)
    assert np.all(np.abs(6.0 * da.astype(np.float64) - ds) <= 4e-7 * np.abs(ds) + 1e-30)
    x, g, a, ap = _case(seed=3, rows=32, dual=True)
    s, sp = (a / np.float32(6)).astype(np.float32), (ap / np.float32(6)).astype(np.float32)
    dx_a, dpre_a, dpost_a = O.fakequant_bwd(x, g, a, ap, amax=True)
    dx_s, dpre_s, dpost_s = O.fakequant_bwd(x, g, s, sp)
    assert np.array_equal(dx_a, dx_s)
    for da_, ds_ in ((dpre_a, dpre_s), (dpost_a, dpost_s)):
        assert np.all(np.abs(6.0 * da_.astype(np.float64) - ds_) <= 4e-7 * np.abs(ds_) + 1e-30)


def test_finite_difference_in_the_post_amax():
    """x~ = q * a_post / 6 is linear in a_post (q fixed by a_pre): with exact
    values the finite difference of L = sum g x~ equals dL/da_post."""
    x, g, a, _ = _case(seed=4, exact=True, rows=16)
    ap = a.copy()
    _, _, dpost = O.fakequant_bwd(x, g, a, ap, amax=True)
    L0 = (g.astype(np.float64) * O.fakequant_fwd(x, a, ap, amax=True)).reshape(-1, 16).sum(axis=1)
    step = (ap * np.float32(2.0 ** -6)).astype(np.float32)     # exact: few significant bits
    L1 = (g.astype(np.float64) * O.fakequant_fwd(x, a, ap + step, amax=True)).reshape(-1, 16).sum(axis=1)
    fd = (L1 - L0) / step.reshape(-1).astype(np.float64)
    d = dpost.reshape(-1).astype(np.float64)
    assert np.all(np.abs(fd - d) <= 1e-6 * np.abs(d) + 1e-12)


def test_tied_is_the_sum_of_dual_gradients():
    x, g, a, _ = _case(seed=5, rows=32)
    _, da = O.fakequant_bwd(x, g, a, amax=True)
    _, dpre, dpost = O.fakequant_bwd(x, g, a, a.copy(), amax=True)
    tot = dpre.astype(np.float64) + dpost
    assert np.all(np.abs(da - tot) <= 1e-5 * np.maximum(np.abs(da), np.abs(tot)) + 1e-12)
