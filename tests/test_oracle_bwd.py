"""Pins for the backward routes of the CPU oracle.

The backward is the vector-Jacobian product of the output equation of the
explainer "Native multi-dimensional subquadratic operators via input-dependent
long convolutions" (section "HyenaND: native-space implicit global kernel",
y[i] = sum_j phi(x[j]) x[j] K[i-j]), returning the gradients of the input and of
the kernel parameters as its autograd pattern does (section "Implementation and
operation patterns", item "Concrete implementation pattern (PyTorch)").  The
pages check gradients by central finite differences (section "Risks and
mitigation strategies", debugging item: (L(t + eps) - L(t - eps)) / (2 eps),
eps = 1e-4), which is one of the pins here.  The others: torch autograd of the
definition written with an explicit Toeplitz gather (no FFT, no hand-derived
chain rule), closed forms for delta kernels and one-hot output gradients,
exact linearity in K, and checks that these pins reject plausible mistakes.
"""
import numpy as np
import pytest
import torch

import oracle


def _case(dims, B=2, C=2, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, C) + tuple(dims)).astype(np.float32)
    dy = rng.standard_normal((B, C) + tuple(dims)).astype(np.float32)
    a = rng.uniform(-1, 1, C).astype(np.float32)
    b = rng.uniform(-1, 1, C).astype(np.float32)
    K = rng.standard_normal((C,) + tuple(2 * n - 1 for n in dims)).astype(np.float32)
    return x, a, b, K, dy


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


def _toeplitz_index(dims):
    """Flat index into K's extents of the offset i - j, for every (i, j) of the grid."""
    grid = np.stack(np.meshgrid(*[np.arange(n) for n in dims], indexing="ij"), -1).reshape(-1, len(dims))
    off = grid[:, None, :] - grid[None, :, :] + (np.asarray(dims) - 1)
    ke = [2 * n - 1 for n in dims]
    flat = np.zeros(off.shape[:2], dtype=np.int64)
    for a, e in enumerate(ke):
        flat = flat * e + off[..., a]
    return torch.from_numpy(flat)


def _autograd(x, a, b, K, dy):
    """Gradients of sum(dy * y) by torch autograd, y from the definition as a gather."""
    B, C = x.shape[:2]
    dims = x.shape[2:]
    L = int(np.prod(dims))
    idx = _toeplitz_index(dims)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    at = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    Kt = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    xs = xt.reshape(B, C, L)
    u = xs * torch.sigmoid(at[None, :, None] * xs + bt[None, :, None])
    T = Kt.reshape(C, -1)[:, idx]  # [C, L, L]: T[c, i, j] = K_c[i - j]
    y = torch.einsum("cij,bcj->bci", T, u)
    loss = (y * torch.tensor(dy, dtype=torch.float64).reshape(B, C, L)).sum()
    gx, ga, gb, gK = torch.autograd.grad(loss, [xt, at, bt, Kt])
    return gx.numpy(), ga.numpy(), gb.numpy(), gK.numpy()


@pytest.mark.parametrize("dims", [(6,), (1,), (3, 4), (4, 1), (2, 3, 2)])
def test_bwd_matches_autograd_of_definition(dims):
    x, a, b, K, dy = _case(dims, seed=1)
    got = oracle.bwd_direct(x, a, b, K, dy)
    want = _autograd(x, a, b, K, dy)
    for g, w, name in zip(got, want, ["dx", "dalpha", "dbeta", "dK"]):
        assert _rel(g, w) < 1e-12, name


@pytest.mark.parametrize("dims", [(16,), (8, 4), (4, 8), (4, 2, 8), (2, 2, 2)])
def test_bwd_fft_matches_direct(dims):
    x, a, b, K, dy = _case(dims, B=3, C=2, seed=2)
    d1 = oracle.bwd_direct(x, a, b, K, dy)
    d2 = oracle.bwd_fft(x, a, b, K, dy)
    for g, w, name in zip(d2, d1, ["dx", "dalpha", "dbeta", "dK"]):
        assert _rel(g, w) < 1e-12, name
    # a subset of channels, in a chosen order
    s = oracle.bwd_fft(x, a, b, K, dy, chans=[1])
    assert _rel(s[0][:, 0], d1[0][:, 1]) < 1e-12 and _rel(s[3][0], d1[3][1]) < 1e-12
    assert abs(s[1][0] - d1[1][1]) < 1e-12 * max(1.0, abs(d1[1][1]))


def test_bwd_points_match_direct():
    dims = (5, 6)
    x, a, b, K, dy = _case(dims, B=2, C=3, seed=3)
    dx, _, _, dK = oracle.bwd_direct(x, a, b, K, dy)
    xp = [(1, 2, 0, 0), (0, 0, 4, 5), (1, 1, 2, 3)]
    kp = [(0, 0, 0), (2, 8, 10), (1, 4, 5), (1, 3, 9)]
    ox, ok = oracle.bwd_points(x, a, b, K, dy, xp, kp)
    assert _rel(ox, [dx[p] for p in xp]) < 1e-12
    assert _rel(ok, [dK[p] for p in kp]) < 1e-12


def _loss(x, a, b, K, dy):
    return float(np.sum(oracle.direct(x, a, b, K) * dy.astype(np.float64)))


def test_finite_differences():
    # Central differences as the explainer prescribes (eps = 1e-4), taken on the
    # fp32 values actually fed to the forward oracle: L(t+) - L(t-) against
    # <grad, t+ - t-> (second-order terms cancel, third-order ones are ~eps^2).
    dims = (4, 5)
    x, a, b, K, dy = _case(dims, B=2, C=2, seed=4)
    dx, da, db, dK = oracle.bwd_direct(x, a, b, K, dy)
    rng = np.random.default_rng(5)
    eps = 1e-4
    v = rng.standard_normal(x.shape)
    xp, xm = (x + eps * v).astype(np.float32), (x - eps * v).astype(np.float32)
    fd = _loss(xp, a, b, K, dy) - _loss(xm, a, b, K, dy)
    an = float(np.sum(dx * (xp.astype(np.float64) - xm.astype(np.float64))))
    assert abs(fd - an) < 1e-6 * abs(an)
    for c in range(2):
        for which, grad in (("alpha", da), ("beta", db)):
            p, m = a.copy(), a.copy()
            if which == "beta":
                p, m = b.copy(), b.copy()
            p[c] += np.float32(eps)
            m[c] -= np.float32(eps)
            if which == "alpha":
                fd = _loss(x, p, b, K, dy) - _loss(x, m, b, K, dy)
            else:
                fd = _loss(x, a, p, K, dy) - _loss(x, a, m, K, dy)
            an = grad[c] * (float(p[c]) - float(m[c]))
            assert abs(fd - an) < 1e-6 * abs(an), (which, c)
    # The loss is linear in K: any step, however large, is exact.
    dK_step = rng.standard_normal(K.shape).astype(np.float32)
    fd = _loss(x, a, b, K + dK_step, dy) - _loss(x, a, b, K, dy)
    an = float(np.sum(dK * (((K + dK_step).astype(np.float64)) - K.astype(np.float64))))
    assert abs(fd - an) < 1e-10 * max(abs(an), 1.0)


def _delta(dims, shift):
    K = np.zeros((1,) + tuple(2 * n - 1 for n in dims), np.float32)
    K[(0,) + tuple(s + n - 1 for s, n in zip(shift, dims))] = 1.0
    return K


@pytest.mark.parametrize("shift", [(0, 0), (2, -1), (-3, 4)])
def test_shifted_delta_kernel(shift):
    # K = delta at s: y[i] = u[i - s], so du[j] = dy[j + s] where j + s is in
    # the grid and exactly 0 elsewhere.
    dims = (5, 6)
    x, a, b, _, dy = _case(dims, B=1, C=1, seed=6)
    K = _delta(dims, shift)
    dx, _, _, _ = oracle.bwd_direct(x, a, b, K, dy)
    du = np.zeros(dims)
    for j in np.ndindex(*dims):
        i = tuple(jj + s for jj, s in zip(j, shift))
        if all(0 <= ii < n for ii, n in zip(i, dims)):
            du[j] = dy[(0, 0) + i]
    x64, a64, b64 = x[0, 0].astype(np.float64), float(a[0]), float(b[0])
    s = 1.0 / (1.0 + np.exp(-(a64 * x64 + b64)))
    want = du * (s + a64 * x64 * s * (1 - s))
    assert np.max(np.abs(dx[0, 0] - want)) < 1e-12


@pytest.mark.parametrize("i0", [(0, 0), (2, 3), (4, 5)])
def test_one_hot_output_gradient(i0):
    # dy = one-hot at i0, B = 1: dK[l] = u[i0 - l] where i0 - l is in the grid.
    dims = (5, 6)
    x, a, b, K, _ = _case(dims, B=1, C=1, seed=7)
    dy = np.zeros_like(x)
    dy[(0, 0) + i0] = 1.0
    _, _, _, dK = oracle.bwd_direct(x, a, b, K, dy)
    u = oracle.gate(x[0, 0], a[0], b[0])
    want = np.zeros(dK.shape[1:])
    for e in np.ndindex(*want.shape):
        l = tuple(ee - (n - 1) for ee, n in zip(e, dims))
        j = tuple(ii - ll for ii, ll in zip(i0, l))
        if all(0 <= jj < n for jj, n in zip(j, dims)):
            want[e] = u[j]
    assert np.max(np.abs(dK[0] - want)) < 1e-12


# ------------------------------------------------------- planted mistakes
def _mut_du_convolution(x, a, b, K, dy):
    # du as a convolution with K instead of a correlation (kernel flipped)
    flip = tuple(range(1, K.ndim))
    return oracle.bwd_direct(x, a, b, np.ascontiguousarray(np.flip(K, flip)), dy)


def _mut_dk_flipped(x, a, b, K, dy):
    dx, da, db, dK = oracle.bwd_direct(x, a, b, K, dy)
    return dx, da, db, np.ascontiguousarray(np.flip(dK, tuple(range(1, dK.ndim))))


def _mut_gate_derivative(x, a, b, K, dy):
    # dx = du * s, dropping the alpha x s (1-s) term
    dx, da, db, dK = oracle.bwd_direct(x, a, b, K, dy)
    xs = x.astype(np.float64)
    s = 1.0 / (1.0 + np.exp(-(a[None, :, None, None] * xs + b[None, :, None, None])))
    return dx / (s + a[None, :, None, None] * xs * s * (1 - s)) * s, da, db, dK


def _mut_dalpha_beta_swapped(x, a, b, K, dy):
    dx, da, db, dK = oracle.bwd_direct(x, a, b, K, dy)
    return dx, db, da, dK


@pytest.mark.parametrize("mutant", [_mut_du_convolution, _mut_dk_flipped, _mut_gate_derivative,
                                    _mut_dalpha_beta_swapped])
def test_pins_reject_mutants(mutant):
    dims = (3, 4)
    x, a, b, K, dy = _case(dims, B=2, C=2, seed=8)
    got = mutant(x, a, b, K, dy)
    want = _autograd(x, a, b, K, dy)
    assert max(_rel(g, w) for g, w in zip(got, want)) > 1e-6, "the autograd pin accepted a planted mistake"


def test_gate_vjp_matches_autograd():
    """oracle.gate_vjp against torch autograd (fp64) of u = sigmoid(a x + b) x:
    the gradient of sum(u * du) with respect to x, a and b; a planted slip (the
    derivative without the a x s (1-s) term) is rejected."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7)).astype(np.float32)
    du = rng.standard_normal((5, 7))
    for a, b in [(0.7, -0.3), (-1.0, 0.5), (0.0, 0.2)]:
        xt = torch.tensor(x.astype(np.float64), requires_grad=True)
        at = torch.tensor(a, dtype=torch.float64, requires_grad=True)
        bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
        (torch.sigmoid(at * xt + bt) * xt * torch.from_numpy(du)).sum().backward()
        dx, da, db = oracle.gate_vjp(x, du, a, b)
        assert _rel(dx, xt.grad.numpy()) < 1e-13
        assert abs(da - float(at.grad)) <= 1e-12 * max(1.0, abs(float(at.grad)))
        assert abs(db - float(bt.grad)) <= 1e-12 * max(1.0, abs(float(bt.grad)))
        s = 1.0 / (1.0 + np.exp(-(a * x.astype(np.float64) + b)))
        if a != 0.0:
            assert _rel(du * s, xt.grad.numpy()) > 1e-3
