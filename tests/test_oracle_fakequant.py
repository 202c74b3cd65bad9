"""Pins of the oracle's scale-learning fake quantization and its
straight-through gradients.  Independent references: torch autograd through
the usual straight-through surrogate (round replaced by identity plus a
detached correction), finite differences where x~ is exactly linear in a
scale, and the tied/dual identity.  CPU only."""
import numpy as np
import pytest
import torch

import oracle as O


def _round_e2m1(y):
    """Nearest E2M1 value with ties to even: torch's ties-to-even round at the
    local grid step (0.5 below 2, 1 below 4, 2 above), saturated at 6."""
    a = y.abs()
    step = torch.where(a < 2, 0.5, torch.where(a < 4, 1.0, 2.0)).to(torch.float64)
    return torch.sign(y) * torch.clamp(torch.round(a / step) * step, max=6.0)


def _autograd_ref(x, g, s_pre, s_post=None):
    """x: [B,16] float64 with x / s exactly representable; returns
    (x~, dx, ds_pre[, ds_post]) from autograd of the STE surrogate."""
    x = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    sp = torch.tensor(s_pre, dtype=torch.float64, requires_grad=True)
    so = sp if s_post is None else torch.tensor(s_post, dtype=torch.float64, requires_grad=True)
    y = x / sp[:, None]
    c = torch.clamp(y, -6.0, 6.0)  # the clamp, its ends included
    r = c + (_round_e2m1(y) - c).detach()  # value of round, derivative of identity
    xq = so[:, None] * r
    (xq * torch.tensor(g, dtype=torch.float64)).sum().backward()
    out = [xq.detach().numpy(), x.grad.numpy(), sp.grad.numpy()]
    if s_post is not None:
        out.append(so.grad.numpy())
    return out


def _exact_blocks(nblk, seed):
    """Blocks whose scales are powers of two, so x / s is exact in both
    binary32 and binary64 and the references see the same y as the oracle.
    Values straddle the clamp at +-6 and hit exact grid points."""
    rng = np.random.default_rng(seed)
    s = 2.0 ** rng.integers(-6, 4, nblk)
    y = rng.choice(np.arange(-64, 65) / 8.0, (nblk, 16))  # multiples of 1/8 in [-8, 8]
    y[:, 0] = rng.choice([-7.0, -6.0, -2.3125, 0.0, 2.3125, 6.0, 7.0], nblk)
    x = (y * s[:, None]).astype(np.float32)
    g = rng.standard_normal((nblk, 16)).astype(np.float32)
    return x, g, s.astype(np.float32)


def test_forward_matches_definition():
    x, g, s = _exact_blocks(64, 0)
    ref = _autograd_ref(x, g, s)[0]
    got = O.fakequant_fwd(x, s)
    assert np.array_equal(got, ref.astype(np.float32))
    s2 = (s * 1.125).astype(np.float32)
    got2 = O.fakequant_fwd(x, s, s2)
    assert np.array_equal(got2, (ref / s[:, None] * s2[:, None]).astype(np.float32))


def test_single_scale_gradients_match_autograd():
    x, g, s = _exact_blocks(128, 1)
    _, dx_ref, ds_ref = _autograd_ref(x, g, s)
    dx, ds = O.fakequant_bwd(x, g, s)
    assert np.array_equal(dx, dx_ref.astype(np.float32))
    assert np.allclose(ds, ds_ref, rtol=1e-6, atol=1e-6 * np.abs(g).sum(1).max())


def test_dual_scale_gradients_match_autograd():
    x, g, s = _exact_blocks(128, 2)
    s_post = (s * 1.125).astype(np.float32)
    _, dx_ref, dpre_ref, dpost_ref = _autograd_ref(x, g, s, s_post)
    dx, dpre, dpost = O.fakequant_bwd(x, g, s, s_post)
    assert np.allclose(dx, dx_ref, rtol=1e-7, atol=0)
    assert np.allclose(dpost, dpost_ref, rtol=1e-7, atol=1e-7)
    assert np.allclose(dpre, dpre_ref, rtol=1e-6, atol=1e-6 * np.abs(dpre_ref).max())


def test_ste_cases_of_the_page(pages):
    c = pages["ste_cases"]
    # one element per block, scale 1: d x~/ds for y below, inside, above
    ys = [-7.0, -6.0, -2.3125, 0.0, 2.3125, 6.0, 7.0]
    x = np.zeros((len(ys), 16), np.float32)
    x[:, 0] = ys
    g = np.zeros_like(x)
    g[:, 0] = 1.0
    s = np.ones(len(ys), np.float32)
    _, ds = O.fakequant_bwd(x, g, s)
    expect = [c["q_min"], -6.0 - (-6.0), -2.0 - (-2.3125), 0.0, 2.0 - 2.3125, 6.0 - 6.0, c["q_max"]]
    assert list(ds) == expect
    dx, _ = O.fakequant_bwd(x, g, s)
    assert list(dx[:, 0]) == [0.0, 1.0, 1.0, 1.0, 1.0, 1.0, 0.0]


def test_clamped_case_is_the_true_derivative():
    """Outside the clamp x~ = +-6 s is linear in s, so a finite difference of
    the forward equals the q_min / q_max case exactly."""
    x = np.zeros((2, 16), np.float32)
    x[0, :] = 10.0
    x[1, :] = -9.0
    s = np.array([1.0, 1.0], np.float32)
    h = np.float32(2.0 ** -10)
    fd = (O.fakequant_fwd(x, s + h) - O.fakequant_fwd(x, s)).sum(1) / h
    g = np.ones_like(x)
    _, ds = O.fakequant_bwd(x, g, s)
    assert np.array_equal(fd, ds)


def test_post_scale_finite_difference():
    """x~ is exactly linear in s_post (pre-scale fixed), so the finite
    difference of sum(g * x~) in s_post equals dL/ds_post."""
    x, g, s = _exact_blocks(32, 3)
    g = np.round(g * 8) / 8  # short mantissas keep the products exact
    h = np.float32(2.0 ** -8)
    so = s.copy()
    f0 = (g.astype(np.float64) * O.fakequant_fwd(x, s, so)).sum(1)
    f1 = (g.astype(np.float64) * O.fakequant_fwd(x, s, so + h * s)).sum(1)
    _, _, dpost = O.fakequant_bwd(x, g, s, so)
    assert np.allclose((f1 - f0) / (h * s), dpost, rtol=0, atol=1e-6)


def test_tied_identity():
    """At s_pre = s_post the single-scale gradient is the sum of the two
    dual-scale gradients (exact in reals)."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((256, 16)) * 0.02).astype(np.float32)
    g = (rng.standard_normal((256, 16)) * 1e-3).astype(np.float32)
    s = (np.abs(x).max(1) / 6 * rng.uniform(0.8, 1.2, 256)).astype(np.float32)
    _, ds = O.fakequant_bwd(x, g, s)
    dx2, dpre, dpost = O.fakequant_bwd(x, g, s, s)
    dx1, _ = O.fakequant_bwd(x, g, s)
    assert np.allclose(ds, dpre.astype(np.float64) + dpost, rtol=1e-5,
                       atol=1e-6 * np.abs(g).sum(1).max())
    assert np.array_equal(dx1, dx2)


def test_zero_scale_block():
    """A zero block scale has no reciprocal; the reading taken is inv = 0, so
    every y = x * inv is a zero (inside the clamp range), every q is zero, the
    forward output is zero for any x, the tied backward passes g through with
    a zero scale gradient, and the dual backward gives zero everywhere
    (r = s_post * inv = 0)."""
    g = np.ones((1, 16), np.float32)
    s = np.zeros(1, np.float32)
    for x in (np.zeros((1, 16), np.float32),
              np.linspace(-3.0, 5.0, 16, dtype=np.float32).reshape(1, 16)):
        assert np.all(O.fakequant_fwd(x, s) == 0)
        assert np.all(O.fakequant_fwd(x, s, np.full(1, 2.0, np.float32)) == 0)
        dx, ds = O.fakequant_bwd(x, g, s)
        assert np.all(dx == 1) and ds[0] == 0
        dx, dpre, dpost = O.fakequant_bwd(x, g, s, np.ones(1, np.float32))
        assert np.all(dx == 0) and dpre[0] == 0 and dpost[0] == 0
