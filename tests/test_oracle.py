"""Pins for the CPU oracle, against facts fixed by the pages and by mathematics.

The operation is the output equation of the explainer "Native multi-dimensional
subquadratic operators via input-dependent long convolutions" (section "HyenaND:
native-space implicit global kernel", y[i] = sum_j phi(x[j]) x[j] K[i-j]) with the
non-circular boundary of the gist.science summary (section "Methodology",
"Boundary handling": zero-pad to twice the grid).  The pages print no worked
example of y, so the pins are: hand-derived closed forms on tiny grids, an
independent pure-Python brute force, delta / shifted-delta / constant / separable
kernel identities, linearity, library cross-checks (torch SiLU, numpy/scipy
FFTs), and checks that these pins reject plausible mistakes.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle


def _rand_case(dims, C=2, B=1, seed=0, alpha=None, beta=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, C) + tuple(dims)).astype(np.float32)
    a = rng.uniform(-1, 1, C).astype(np.float32) if alpha is None else np.full(C, alpha, np.float32)
    b = rng.uniform(-1, 1, C).astype(np.float32) if beta is None else np.full(C, beta, np.float32)
    K = rng.standard_normal((C,) + tuple(2 * n - 1 for n in dims)).astype(np.float32)
    return x, a, b, K


def _brute(x, alpha, beta, K):
    """Pure-Python quadruple loop over the output equation (independent of oracle.c)."""
    B, C = x.shape[:2]
    dims = x.shape[2:]
    y = np.zeros(x.shape, dtype=np.float64)
    grid = list(itertools.product(*[range(n) for n in dims]))
    for b in range(B):
        for c in range(C):
            u = {}
            for j in grid:
                v = float(x[(b, c) + j])
                u[j] = v / (1.0 + math.exp(-(float(alpha[c]) * v + float(beta[c]))))
            for i in grid:
                acc = 0.0
                for j in grid:
                    kidx = tuple(ia - ja + n - 1 for ia, ja, n in zip(i, j, dims))
                    acc += u[j] * float(K[(c,) + kidx])
                y[(b, c) + i] = acc
    return y


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- closed forms

def test_hand_worked_2x2():
    # alpha = beta = 0 makes the gate exactly 1/2, so u = x / 2 = [[1,2],[3,4]].
    # K[d0+1][d1+1] = [[1,2,3],[4,5,6],[7,8,9]].  By hand:
    # y00 = 1*5 + 2*4 + 3*2 + 4*1 = 23      y01 = 1*6 + 2*5 + 3*3 + 4*2 = 33
    # y10 = 1*8 + 2*7 + 3*5 + 4*4 = 53      y11 = 1*9 + 2*8 + 3*6 + 4*5 = 63
    x = np.array([[[[2, 4], [6, 8]]]], np.float32)
    K = np.arange(1, 10, dtype=np.float32).reshape(1, 3, 3)
    z = np.zeros(1, np.float32)
    want = np.array([[[[23, 33], [53, 63]]]], np.float64)
    assert np.array_equal(oracle.direct(x, z, z, K), want)
    assert np.max(np.abs(oracle.fftconv(x, z, z, K) - want)) < 1e-12


def test_hand_worked_1d_orientation():
    # u = x/2 = [1,2,3,4]; K over offsets -3..3 = [1, 10, ..., 10^6] (offset 0 -> 1000).
    # y[i] = sum_j u[j] K[i-j]: y0 = 1*1000 + 2*100 + 3*10 + 4*1 = 1234, and every step
    # of i multiplies by ten: 12340, 123400, 1234000.  A correlation reverses the
    # digits (4321, ...); a circular wrap adds terms from the far end.
    x = np.array([[[2, 4, 6, 8]]], np.float32)
    K = (10.0 ** np.arange(7)).astype(np.float32)[None]
    z = np.zeros(1, np.float32)
    want = np.array([[[1234, 12340, 123400, 1234000]]], np.float64)
    assert np.array_equal(oracle.direct(x, z, z, K), want)
    assert np.max(np.abs(oracle.fftconv(x, z, z, K) - want)) < 1e-7


def test_gate_is_silu_and_constant():
    x = np.random.default_rng(1).standard_normal(1000).astype(np.float32) * 4
    silu = torch.nn.functional.silu(torch.from_numpy(x).double()).numpy()
    assert np.max(np.abs(oracle.gate(x, 1.0, 0.0) - silu)) < 1e-14
    beta = 0.37
    const = x.astype(np.float64) / (1.0 + np.exp(-beta))
    assert np.max(np.abs(oracle.gate(x, 0.0, beta) - const)) < 1e-14


# ------------------------------------------------------- brute force, O1 vs O2

@pytest.mark.parametrize("dims", [(5,), (16,), (3, 4), (8, 8), (2, 3, 4), (4, 4, 4)])
def test_direct_matches_pure_python(dims):
    x, a, b, K = _rand_case(dims, C=2, B=2, seed=len(dims) * 7 + dims[0])
    assert _rel(oracle.direct(x, a, b, K), _brute(x, a, b, K)) < 1e-13


@pytest.mark.parametrize("dims", [(2,), (64,), (8, 16), (16, 16), (32, 8), (4, 8, 4), (8, 8, 8), (2, 4, 16)])
def test_fft_route_matches_direct(dims):
    x, a, b, K = _rand_case(dims, C=3, B=2, seed=sum(dims))
    yd = oracle.direct(x, a, b, K)
    yf = oracle.fftconv(x, a, b, K)
    assert _rel(yf, yd) < 1e-12
    # Subsets of pairs come back in the order asked for.
    sub = oracle.fftconv(x, a, b, K, pairs=[5, 0, 3])
    assert _rel(sub, yd.reshape((6,) + dims)[[5, 0, 3]]) < 1e-12


def test_direct_points_match_direct():
    dims = (8, 4, 16)
    x, a, b, K = _rand_case(dims, C=3, B=2, seed=11)
    yd = oracle.direct(x, a, b, K)
    pts = np.array([[1, 2, 7, 3, 15], [0, 0, 0, 0, 0], [1, 2, 0, 0, 1], [0, 1, 4, 2, 9]], np.int64)
    got = oracle.direct_points(x, a, b, K, pts)
    want = np.array([yd[tuple(p)] for p in pts])
    assert np.max(np.abs(got - want)) < 1e-12 * np.max(np.abs(yd))


# ------------------------------------------------------------ kernel identities

def _delta(dims, shift, C=1):
    K = np.zeros((C,) + tuple(2 * n - 1 for n in dims), np.float32)
    K[(slice(None),) + tuple(n - 1 + s for n, s in zip(dims, shift))] = 1.0
    return K


def _shifted(u, shift):
    """u moved by +shift with zero fill: out[i] = u[i - s] when i - s is inside."""
    out = np.zeros_like(u)
    src = tuple(slice(max(0, -s), n - max(0, s)) for n, s in zip(u.shape, shift))
    dst = tuple(slice(max(0, s), n - max(0, -s)) for n, s in zip(u.shape, shift))
    out[dst] = u[src]
    return out


SHIFT_CASES = [((16,), (0,)), ((16,), (5,)), ((16,), (-15,)), ((8, 16), (3, -7)), ((8, 16), (-7, 15)),
               ((4, 8, 8), (1, -2, 3)), ((4, 8, 8), (-3, 7, -7))]


@pytest.mark.parametrize("route", ["direct", "fft"])
@pytest.mark.parametrize("dims,shift", SHIFT_CASES)
def test_shifted_delta(route, dims, shift):
    x, a, b, _ = _rand_case(dims, C=1, seed=3)
    K = _delta(dims, shift)
    fn = oracle.direct if route == "direct" else oracle.fftconv
    y = fn(x, a, b, K)[0, 0]
    u = oracle.gate(x[0, 0], a[0], b[0])
    want = _shifted(u, shift)
    assert np.max(np.abs(y - want)) < 1e-12
    # Outside the shifted support the output is exactly zero for the direct sum
    # (non-circular boundary: nothing wraps around).
    if route == "direct":
        assert np.all(y[want == 0] == 0)


@pytest.mark.parametrize("dims", [(32,), (8, 8), (4, 4, 4)])
def test_constant_kernel_sums(dims):
    x, a, b, _ = _rand_case(dims, C=1, seed=5)
    K = np.ones((1,) + tuple(2 * n - 1 for n in dims), np.float32)
    u = oracle.gate(x[0, 0], a[0], b[0])
    for fn in (oracle.direct, oracle.fftconv):
        y = fn(x, a, b, K)[0, 0]
        assert np.max(np.abs(y - u.sum())) < 1e-11


def test_separable_kernel_is_iterated_1d_convolution():
    # K(d0, d1) = k0(d0) * k1(d1) with short dyadic factors, so the fp32 outer
    # product is exact and the 2-D convolution must equal two 1-D full
    # convolutions (numpy.convolve) cropped to [n-1, 2n-1).
    dims = (8, 16)
    rng = np.random.default_rng(9)
    k0 = rng.integers(-8, 9, 15) / 8.0
    k1 = rng.integers(-8, 9, 31) / 4.0
    K = np.outer(k0, k1).astype(np.float32)[None]
    assert np.array_equal(K[0].astype(np.float64), np.outer(k0, k1))
    x, a, b, _ = _rand_case(dims, C=1, seed=9)
    u = oracle.gate(x[0, 0], a[0], b[0])
    t = np.array([np.convolve(row, k1, mode="full")[15:31] for row in u])          # axis 1
    ref = np.array([np.convolve(col, k0, mode="full")[7:15] for col in t.T]).T    # axis 0
    for fn in (oracle.direct, oracle.fftconv):
        assert _rel(fn(x, a, b, K)[0, 0], ref) < 1e-12


def test_linearity_in_kernel_and_input():
    dims = (8, 8)
    x, a, b, K1 = _rand_case(dims, C=2, seed=13)
    _, _, _, K2 = _rand_case(dims, C=2, seed=14)
    s = np.float32(0.5)
    for fn in (oracle.direct, oracle.fftconv):
        lhs = fn(x, a, b, (K1 + s * K2).astype(np.float32))
        rhs = fn(x, a, b, K1) + fn(x, a, b, (s * K2).astype(np.float32))
        assert _rel(lhs, rhs) < 1e-6  # K1 + s*K2 is rounded to fp32 once
    # alpha = 0 makes the gate a constant, so y is linear in x.
    z = np.zeros(2, np.float32)
    x2, _, _, _ = _rand_case(dims, C=2, seed=15)
    for fn in (oracle.direct, oracle.fftconv):
        lhs = fn((x + x2).astype(np.float32), z, b, K1)
        rhs = fn(x, z, b, K1) + fn(x2, z, b, K1)
        assert _rel(lhs, rhs) < 1e-6


def test_shift_equivariance():
    # A signal supported in a box, moved by s inside the grid, gives an output
    # moved by s wherever both outputs are defined.
    dims = (16, 16)
    rng = np.random.default_rng(21)
    x = np.zeros((1, 1) + dims, np.float32)
    x[0, 0, 2:6, 3:8] = rng.standard_normal((4, 5))
    s = (5, 4)
    xs = np.zeros_like(x)
    xs[0, 0, 2 + s[0]:6 + s[0], 3 + s[1]:8 + s[1]] = x[0, 0, 2:6, 3:8]
    _, a, b, K = _rand_case(dims, C=1, seed=22)
    for fn in (oracle.direct, oracle.fftconv):
        y = fn(x, a, b, K)[0, 0]
        ys = fn(xs, a, b, K)[0, 0]
        assert np.max(np.abs(ys[s[0]:, s[1]:] - y[:16 - s[0], :16 - s[1]])) < 1e-11


def test_matches_scipy_fftconvolve():
    scipy_signal = pytest.importorskip("scipy.signal")
    for dims in [(64,), (16, 32), (8, 8, 16)]:
        x, a, b, K = _rand_case(dims, C=2, B=1, seed=31)
        y = oracle.fftconv(x, a, b, K)
        for c in range(2):
            u = oracle.gate(x[0, c], a[c], b[c])
            full = scipy_signal.fftconvolve(u, K[c].astype(np.float64), mode="full")
            ref = full[tuple(slice(n - 1, 2 * n - 1) for n in dims)]
            assert _rel(y[0, c], ref) < 1e-12


# ------------------------------------------------------------------ spectrum

def _wrap_place_numpy(Kc, dims):
    N = tuple(2 * n for n in dims)
    buf = np.zeros(N, np.float64)
    buf[tuple(slice(0, 2 * n - 1) for n in dims)] = Kc
    return np.roll(buf, shift=tuple(-(n - 1) for n in dims), axis=tuple(range(len(dims))))


@pytest.mark.parametrize("dims", [(16,), (8, 4), (4, 8, 4)])
def test_kernel_spectrum_pins(dims):
    _, _, _, K = _rand_case(dims, C=2, seed=41)
    S = oracle.kernel_spectrum(K, dims)
    ax = tuple(range(1, len(dims) + 1))
    for c in range(2):
        wp = _wrap_place_numpy(K[c].astype(np.float64), dims)
        # The slot n of every axis stays empty (the pad is never reached).
        for a, n in enumerate(dims):
            assert np.all(np.take(wp, n, axis=a) == 0)
        assert np.max(np.abs(S[c] - np.fft.fftn(wp))) < 1e-10
        # Real kernel: Hermitian spectrum; DC is the kernel sum; inverse restores it.
        neg = tuple((-np.arange(2 * n)) % (2 * n) for n in dims)
        assert np.max(np.abs(S[c][np.ix_(*neg)] - np.conj(S[c]))) < 1e-10
        assert abs(S[c].flat[0] - K[c].astype(np.float64).sum()) < 1e-10
        assert np.max(np.abs(np.fft.ifftn(S[c]).real - wp)) < 1e-12
    assert S.shape == (2,) + tuple(2 * n for n in dims)
    del ax


# ------------------------------------------------------ the pins catch mistakes

def _correlation(x, a, b, K):
    # Mistake: correlation instead of convolution (kernel index j - i).
    return oracle.direct(x, a, b, np.ascontiguousarray(K[(slice(None),) + (slice(None, None, -1),) * (K.ndim - 1)]))


def _circular(x, a, b, K):
    # Mistake: no zero padding (circular convolution of size n).
    B, C = x.shape[:2]
    dims = x.shape[2:]
    y = np.empty(x.shape)
    for bb in range(B):
        for c in range(C):
            u = oracle.gate(x[bb, c], a[c], b[c])
            kc = np.zeros(dims)
            for idx in itertools.product(*[range(2 * n - 1) for n in dims]):
                kc[tuple((i - (n - 1)) % n for i, n in zip(idx, dims))] += K[(c,) + idx]
            y[bb, c] = np.real(np.fft.ifftn(np.fft.fftn(u) * np.fft.fftn(kc)))
    return y


def _transposed(x, a, b, K):
    # Mistake: kernel axes swapped.
    return oracle.direct(x, a, b, np.ascontiguousarray(np.swapaxes(K, 1, 2)))


def _no_gate(x, a, b, K):
    # Mistake: the gate dropped (y = K * x).
    big = np.full_like(a, 0.0)
    return oracle.direct(x, big, np.full_like(b, 80.0), K)


@pytest.mark.parametrize("mutant", [_correlation, _circular, _transposed, _no_gate])
def test_pins_reject_mutants(mutant):
    dims = (8, 8)
    x, a, b, _ = _rand_case(dims, C=1, seed=3)
    u = oracle.gate(x[0, 0], a[0], b[0])
    fails = 0
    for shift in [(3, -5), (-2, 7)]:
        K = _delta(dims, shift)
        if mutant is _transposed:
            K = _delta(dims, shift)
        y = mutant(x, a, b, K)[0, 0]
        if np.max(np.abs(y - _shifted(u, shift))) > 1e-9:
            fails += 1
    assert fails > 0, "the shifted-delta pin accepted a planted mistake"


# ------------------------------------------------ input-dependent kernels

def test_per_sample_kernels_match_brute_force():
    """One kernel per (b, c) (the summary's kernels conditioned on the input
    sample): the per-sample routes against the pure-Python brute force run
    with each batch entry's own kernels, and identical kernels across the
    batch reduce to the shared-kernel oracle."""
    dims = (3, 4)
    x, a, b, _ = _rand_case(dims, C=2, B=3, seed=21)
    rng = np.random.default_rng(22)
    K = rng.standard_normal((3, 2) + tuple(2 * n - 1 for n in dims)).astype(np.float32)
    want = np.concatenate([_brute(x[i:i + 1], a, b, K[i]) for i in range(3)], axis=0)
    assert _rel(oracle.direct_per_sample(x, a, b, K), want) < 1e-12
    dims2 = (4, 8)
    x2, a2, b2, K2 = _rand_case(dims2, C=2, B=2, seed=23)
    Kb = np.stack([K2, K2 * 0.5 + 1.0])
    got = oracle.fftconv_per_sample(x2, a2, b2, Kb)
    assert _rel(got[0], oracle.direct(x2[:1], a2, b2, K2)[0]) < 1e-12
    assert _rel(got[1], oracle.direct(x2[1:], a2, b2, Kb[1])[0]) < 1e-12


def _autograd_per_sample(x, a, b, K, dy):
    """Gradients of sum(dy * y), y[b,c,i] = sum_j u[b,c,j] K[b,c][i-j] written
    as a gather of each sample's Toeplitz matrix, by torch autograd (fp64)."""
    import torch

    B, C = x.shape[:2]
    dims = x.shape[2:]
    L = int(np.prod(dims))
    grid = np.stack(np.meshgrid(*[np.arange(n) for n in dims], indexing="ij"), -1).reshape(-1, len(dims))
    off = grid[:, None, :] - grid[None, :, :] + (np.asarray(dims) - 1)
    flat = np.zeros(off.shape[:2], dtype=np.int64)
    for ax, n in enumerate(dims):
        flat = flat * (2 * n - 1) + off[..., ax]
    idx = torch.from_numpy(flat)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    at = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
    Kt = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    xs = xt.reshape(B, C, L)
    u = xs * torch.sigmoid(at[None, :, None] * xs + bt[None, :, None])
    T = Kt.reshape(B, C, -1)[:, :, idx]
    y = torch.einsum("bcij,bcj->bci", T, u)
    loss = (y * torch.tensor(dy, dtype=torch.float64).reshape(B, C, L)).sum()
    return [g.numpy() for g in torch.autograd.grad(loss, [xt, at, bt, Kt])]


@pytest.mark.parametrize("dims", [(5,), (3, 4), (2, 3, 2)])
def test_per_sample_bwd_matches_autograd_of_definition(dims):
    """The per-sample backward (dK per (b, c), dalpha / dbeta summed over the
    batch) against torch autograd of the definition with each sample's kernels;
    the FFT route against the direct one; a planted mistake (dK summed over the
    batch, the shared-kernel gradient) fails."""
    B, C = 3, 2
    x, a, b, _ = _rand_case(dims, C=C, B=B, seed=41)
    rng = np.random.default_rng(42)
    K = rng.standard_normal((B, C) + tuple(2 * n - 1 for n in dims)).astype(np.float32)
    dy = rng.standard_normal(x.shape).astype(np.float32)
    want = _autograd_per_sample(x, a, b, K, dy)
    got = oracle.bwd_direct_per_sample(x, a, b, K, dy)
    for g, w in zip(got, want):
        assert g.shape == w.shape
        assert _rel(g, w) < 1e-12
    shared = np.broadcast_to(got[3].sum(axis=0), got[3].shape)
    assert _rel(shared, want[3]) > 1e-3


@pytest.mark.parametrize("dims", [(16,), (4, 8), (2, 4, 8)])
def test_per_sample_bwd_fft_matches_direct(dims):
    B, C = 3, 2
    x, a, b, _ = _rand_case(dims, C=C, B=B, seed=43)
    rng = np.random.default_rng(44)
    K = rng.standard_normal((B, C) + tuple(2 * n - 1 for n in dims)).astype(np.float32)
    dy = rng.standard_normal(x.shape).astype(np.float32)
    for g, w in zip(oracle.bwd_fft_per_sample(x, a, b, K, dy), oracle.bwd_direct_per_sample(x, a, b, K, dy)):
        assert _rel(g, w) < 1e-12
