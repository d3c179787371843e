"""Pins for the circular mode of the CPU oracle.

The gist.science summary ("Methodology", "Boundary handling") gives the method
circular convolutions for periodic physical systems next to the zero-padded
non-circular ones.  On a periodic grid the output equation of the explainer
("HyenaND: native-space implicit global kernel", y[i] = sum_j phi(x[j]) x[j]
K[i-j]) takes the offset i - j modulo n, so K lives on n offsets per axis,
stored with index m = offset mod n.  Pins: an independent pure-Python brute
force, circularly shifted deltas (np.roll), a constant kernel (closed form),
numpy's FFT (a library routine), the identity with the non-circular mode for
the periodically extended kernel, and planted mistakes that these reject.
"""
import itertools
import math

import numpy as np
import pytest

import oracle


def _case(dims, B=2, C=2, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, C) + tuple(dims)).astype(np.float32)
    a = rng.uniform(-1, 1, C).astype(np.float32)
    b = rng.uniform(-1, 1, C).astype(np.float32)
    K = rng.standard_normal((C,) + tuple(dims)).astype(np.float32)
    return x, a, b, K


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _brute(x, alpha, beta, K):
    B, C = x.shape[:2]
    dims = x.shape[2:]
    y = np.zeros(x.shape)
    grid = list(itertools.product(*[range(n) for n in dims]))
    for b in range(B):
        for c in range(C):
            u = {j: float(x[(b, c) + j]) / (1.0 + math.exp(-(float(alpha[c]) * float(x[(b, c) + j]) + float(beta[c]))))
                 for j in grid}
            for i in grid:
                y[(b, c) + i] = sum(u[j] * float(K[(c,) + tuple((ii - jj) % n for ii, jj, n in zip(i, j, dims))])
                                    for j in grid)
    return y


@pytest.mark.parametrize("dims", [(5,), (3, 4), (2, 3, 2)])
def test_direct_matches_pure_python(dims):
    x, a, b, K = _case(dims, seed=1)
    assert _rel(oracle.direct_circ(x, a, b, K), _brute(x, a, b, K)) < 1e-12


@pytest.mark.parametrize("dims", [(16,), (8, 4), (4, 16), (4, 2, 8), (2, 2, 2)])
def test_fft_route_matches_direct(dims):
    x, a, b, K = _case(dims, B=2, C=3, seed=2)
    assert _rel(oracle.fftconv_circ(x, a, b, K), oracle.direct_circ(x, a, b, K)) < 1e-12


@pytest.mark.parametrize("dims,shift", [((8,), (3,)), ((4, 8), (1, -3)), ((4, 4, 8), (-1, 2, 5))])
def test_shifted_delta_rolls_with_wrap(dims, shift):
    x, a, b, _ = _case(dims, B=1, C=1, seed=3)
    K = np.zeros((1,) + dims, np.float32)
    K[(0,) + tuple(s % n for s, n in zip(shift, dims))] = 1.0
    u = oracle.gate(x[0, 0], a[0], b[0])
    want = np.roll(u, shift, axis=tuple(range(len(dims))))
    for route in (oracle.direct_circ, oracle.fftconv_circ):
        assert np.max(np.abs(route(x, a, b, K)[0, 0] - want)) < 1e-12


def test_constant_kernel_sums():
    dims = (4, 8)
    x, a, b, _ = _case(dims, B=1, C=1, seed=4)
    K = np.ones((1,) + dims, np.float32)
    u = oracle.gate(x[0, 0], a[0], b[0])
    assert np.max(np.abs(oracle.direct_circ(x, a, b, K)[0, 0] - u.sum())) < 1e-12


@pytest.mark.parametrize("dims", [(8,), (4, 8), (2, 4, 4)])
def test_matches_numpy_fft(dims):
    x, a, b, K = _case(dims, B=1, C=2, seed=5)
    for c in range(2):
        u = oracle.gate(x[0, c], a[c], b[c])
        want = np.fft.ifftn(np.fft.fftn(u) * np.fft.fftn(K[c].astype(np.float64))).real
        assert _rel(oracle.fftconv_circ(x, a, b, K)[0, c], want) < 1e-12


@pytest.mark.parametrize("dims", [(6,), (3, 4), (2, 3, 4)])
def test_equals_noncircular_mode_with_periodic_extension(dims):
    # For i, j in the grid, i - j lies in [-(n-1), n-1], so the circular sum is
    # the non-circular one with K'[delta] = K[delta mod n].
    x, a, b, K = _case(dims, B=2, C=2, seed=6)
    idx = np.ix_(*[np.arange(-(n - 1), n) % n for n in dims])
    Kp = np.stack([K[c][idx] for c in range(K.shape[0])])
    assert _rel(oracle.direct_circ(x, a, b, K), oracle.direct(x, a, b, Kp)) < 1e-12


def _mut_noncircular(x, a, b, K):
    # zero outside the grid instead of wrapping: offsets beyond n-1 dropped
    dims = x.shape[2:]
    Kp = np.zeros((K.shape[0],) + tuple(2 * n - 1 for n in dims), np.float32)
    for c in range(K.shape[0]):
        for m in np.ndindex(*dims):
            Kp[(c,) + tuple(mm + n - 1 for mm, n in zip(m, dims))] = K[(c,) + m]
    return oracle.direct(x, a, b, Kp)


def _mut_correlation(x, a, b, K):
    ax = tuple(range(1, K.ndim))
    return oracle.direct_circ(x, a, b, np.ascontiguousarray(np.roll(np.flip(K, ax), 1, ax)))


@pytest.mark.parametrize("mutant", [_mut_noncircular, _mut_correlation])
def test_pins_reject_mutants(mutant):
    dims = (4, 8)
    x, a, b, _ = _case(dims, B=1, C=1, seed=7)
    u = oracle.gate(x[0, 0], a[0], b[0])
    fails = 0
    for shift in [(1, -3), (2, 5)]:
        K = np.zeros((1,) + dims, np.float32)
        K[(0,) + tuple(s % n for s, n in zip(shift, dims))] = 1.0
        if np.max(np.abs(mutant(x, a, b, K)[0, 0] - np.roll(u, shift, axis=(0, 1)))) > 1e-9:
            fails += 1
    assert fails > 0


# ------------------------------------------------------------------ backward

def _autograd_circ(x, a, b, K, dy):
    """Gradients of sum(dy * y) by torch autograd, y the circular sum as a gather."""
    import torch

    B, C = x.shape[:2]
    dims = x.shape[2:]
    L = int(np.prod(dims))
    grid = np.stack(np.meshgrid(*[np.arange(n) for n in dims], indexing="ij"), -1).reshape(-1, len(dims))
    off = (grid[:, None, :] - grid[None, :, :]) % np.asarray(dims)
    flat = np.zeros(off.shape[:2], dtype=np.int64)
    for ax, n in enumerate(dims):
        flat = flat * n + off[..., ax]
    idx = torch.from_numpy(flat)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    at = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    Kt = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    xs = xt.reshape(B, C, L)
    u = xs * torch.sigmoid(at[None, :, None] * xs + bt[None, :, None])
    T = Kt.reshape(C, -1)[:, idx]
    y = torch.einsum("cij,bcj->bci", T, u)
    loss = (y * torch.tensor(dy, dtype=torch.float64).reshape(B, C, L)).sum()
    return [g.numpy() for g in torch.autograd.grad(loss, [xt, at, bt, Kt])]


@pytest.mark.parametrize("dims", [(6,), (3, 4), (2, 3, 2)])
def test_bwd_matches_autograd_of_definition(dims):
    x, a, b, K = _case(dims, B=2, C=2, seed=30)
    dy = np.random.default_rng(31).standard_normal(x.shape).astype(np.float32)
    got = oracle.bwd_direct_circ(x, a, b, K, dy)
    for g, w in zip(got, _autograd_circ(x, a, b, K, dy)):
        assert _rel(g, w) < 1e-12


@pytest.mark.parametrize("dims", [(16,), (8, 4), (4, 2, 8)])
def test_bwd_fft_matches_direct(dims):
    x, a, b, K = _case(dims, B=3, C=2, seed=32)
    dy = np.random.default_rng(33).standard_normal(x.shape).astype(np.float32)
    d1 = oracle.bwd_direct_circ(x, a, b, K, dy)
    d2 = oracle.bwd_fft_circ(x, a, b, K, dy)
    for g, w in zip(d2, d1):
        assert _rel(g, w) < 1e-12


def test_bwd_finite_differences():
    # The explainer's central differences (eps = 1e-4) on x, and exact linearity in K.
    dims = (4, 4)
    x, a, b, K = _case(dims, B=2, C=2, seed=34)
    rng = np.random.default_rng(35)
    dy = rng.standard_normal(x.shape).astype(np.float32)
    dx, _, _, dK = oracle.bwd_direct_circ(x, a, b, K, dy)
    loss = lambda xx, KK: float(np.sum(oracle.direct_circ(xx, a, b, KK) * dy.astype(np.float64)))
    v = rng.standard_normal(x.shape)
    xp, xm = (x + 1e-4 * v).astype(np.float32), (x - 1e-4 * v).astype(np.float32)
    an = float(np.sum(dx * (xp.astype(np.float64) - xm.astype(np.float64))))
    assert abs(loss(xp, K) - loss(xm, K) - an) < 1e-6 * abs(an)
    step = rng.standard_normal(K.shape).astype(np.float32)
    an = float(np.sum(dK * ((K + step).astype(np.float64) - K.astype(np.float64))))
    assert abs(loss(x, K + step) - loss(x, K) - an) < 1e-10 * max(abs(an), 1.0)


def test_bwd_pins_reject_planted_mistakes():
    dims = (4, 4)
    x, a, b, K = _case(dims, B=1, C=1, seed=36)
    dy = np.random.default_rng(37).standard_normal(x.shape).astype(np.float32)
    want = _autograd_circ(x, a, b, K, dy)
    dx, da, db, dK = oracle.bwd_direct_circ(x, a, b, K, dy)
    ax = tuple(range(1, dK.ndim))
    mutants = [
        (dx, da, db, np.roll(np.flip(dK, ax), 1, ax)),              # dK with the offset sign flipped
        oracle.bwd_direct_circ(x, a, b, np.ascontiguousarray(np.roll(np.flip(K, ax), 1, ax)), dy),  # du a convolution
    ]
    for m in mutants:
        assert max(_rel(g, w) for g, w in zip(m, want)) > 1e-6
