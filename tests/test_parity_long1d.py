"""GPU parity of long 1-D convolutions (n > 1024: the four-step path) against
the fp64 oracle.

The gist.science summary ("Results", genomics) reports throughput up to 10M
tokens for 1-D signals; here the zero-padded length N = 2n is factored as
N1 x N2 (column transforms, twiddle, row transforms with the spectrum product)
for n up to 2^23 (rows of 4096 points beyond N = 2^22).  Bar as for the other forwards: max|y_gpu - y_ref| / max|y_ref|
<= 1e-4 (fp32 I/O), <= 2e-2 (bf16 I/O).  Whole signals against the oracle's
FFT route (O2) and sampled outputs against the direct sum (O1).  The backward
(dx, dalpha, dbeta, dK) as for the other backwards: <= 1e-4 for fp32 I/O; bf16
I/O: dx <= 2e-2, the fp32 parameter and kernel gradients <= 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dimensional_fft_long_amd as H

    H.get_lib()
    return H


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def _run(H, dims, B, C, dtype, seed, per_sample=False, workspace=None):
    dev = torch.device("cuda:0")
    p = synth.draw_params(dims, C, seed)
    x = synth.draw_x(p.rng, B, C, dims, dtype)
    K = synth.kernel_channels(dims, p, device=dev)
    al, be = torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev)
    if per_sample:
        scale = torch.linspace(0.5, 1.5, B, device=dev).reshape(B, 1, 1)
        Kb = (K.unsqueeze(0) * scale).contiguous()
        y = H.fftconv_fwd_per_sample(x.to(dev), al, be, H.kernel_spectrum_per_sample(Kb), workspace=workspace)
        K = Kb
    else:
        y = H.fftconv_fwd(x.to(dev), al, be, H.kernel_spectrum(K), workspace=workspace)
    torch.cuda.synchronize()
    return x.float().numpy(), p, K.cpu().numpy(), y.float().cpu().numpy()


@pytest.mark.parametrize("n,B,C,dtype", [(2048, 2, 3, "f32"), (4096, 1, 2, "bf16"), (8192, 3, 2, "f32"),
                                         (1 << 16, 2, 2, "f32"), (1 << 18, 1, 2, "bf16"), (1 << 20, 1, 2, "f32"),
                                         (1 << 22, 1, 1, "f32"), (1 << 23, 1, 1, "bf16"), (1 << 24, 1, 1, "f32")],
                         ids=lambda v: str(v))
def test_matches_fft_oracle(H, n, B, C, dtype):
    x, p, K, y = _run(H, (n,), B, C, dtype, seed=200 + n % 97 + B)
    ref = oracle.fftconv(x, p.alpha, p.beta, K)
    assert np.all(np.isfinite(y))
    assert _rel(y, ref) <= TOL[dtype]


def test_sampled_outputs_match_direct_sum(H):
    n = 1 << 14
    x, p, K, y = _run(H, (n,), 2, 2, "f32", seed=7)
    pts = synth.sample_points((n,), 2, 2, [(0, 0), (1, 1)], 24, seed=7)
    ref = oracle.direct_points(x, p.alpha, p.beta, K, pts)
    got = np.array([y[tuple(r)] for r in pts])
    assert _rel(got, ref) <= 1e-4


def test_per_sample_kernels(H):
    n = 1 << 13
    x, p, Kb, y = _run(H, (n,), 3, 2, "f32", seed=8, per_sample=True)
    ref = oracle.direct_per_sample(x, p.alpha, p.beta, Kb)
    assert _rel(y, ref) <= 1e-4


def test_every_chunking_gives_the_same_output(H):
    n, B, C = 1 << 12, 2, 5
    minb = H.workspace_bytes(B, C, (n,), torch.float32, minimum=True)
    outs = [_run(H, (n,), B, C, "f32", seed=9, workspace=torch.empty(k * minb, dtype=torch.uint8, device="cuda"))[3]
            for k in (1, 2, C)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.timeout(600)
def test_workload_16m_tokens(H):
    """2^24 tokens (the summary's 10M-token context zero-extended to a power
    of two; 8192-point rows), bf16, both channels against the FFT oracle, and
    sampled outputs (corners, centre, random) against the direct sum."""
    wl = {w.name: w for w in synth.WORKLOADS}["1d_16777216_b1_c2_bf16"]
    x, p, K, y = _run(H, wl.dims, wl.B, wl.C, wl.dtype, seed=wl.seed)
    assert np.all(np.isfinite(y))
    for c in range(wl.C):
        ref = oracle.fftconv(x[:, c:c + 1], p.alpha[c:c + 1], p.beta[c:c + 1], K[c:c + 1])
        assert _rel(y[:, c], ref[:, 0]) <= TOL[wl.dtype], c
    pts = synth.sample_points(wl.dims, wl.B, wl.C, [(0, 0), (0, 1)], 16, seed=wl.seed, edges=True)
    ref = oracle.direct_points(x, p.alpha, p.beta, K, pts)
    assert _rel(np.array([y[tuple(r)] for r in pts]), ref) <= TOL[wl.dtype]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("idx", [5, 6])
def test_workload_full_size(H, idx):
    """The 2M-token (8 channels) and 8M-token (4 channels) bf16 workloads at full
    size: the first and last channel against the FFT oracle."""
    wl = synth.WORKLOADS[idx]
    x, p, K, y = _run(H, wl.dims, wl.B, wl.C, wl.dtype, seed=wl.seed)
    for c in (0, wl.C - 1):
        ref = oracle.fftconv(x[:, c:c + 1], p.alpha[c:c + 1], p.beta[c:c + 1], K[c:c + 1])
        assert _rel(y[:, c], ref[:, 0]) <= TOL[wl.dtype], c


# ------------------------------------------------------------------ backward

TOL_DX = {"f32": 1e-4, "bf16": 2e-2}
TOL_PARAM = {"f32": 1e-4, "bf16": 1e-3}


def _run_bwd(H, dims, B, C, dtype, seed, with_dK=True, workspace=None, per_sample=False):
    dev = torch.device("cuda:0")
    p = synth.draw_params(dims, C, seed)
    x = synth.draw_x(p.rng, B, C, dims, dtype)
    dy = synth.draw_dy(dims, B, C, dtype, seed)
    K = synth.kernel_channels(dims, p, device=dev)
    al, be = torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev)
    if per_sample:
        scale = torch.linspace(0.5, 1.5, B, device=dev).reshape(B, 1, 1)
        K = (K.unsqueeze(0) * scale).contiguous()
        out = H.fftconv_bwd_per_sample(x.to(dev), al, be, H.kernel_spectrum_per_sample(K), dy.to(dev),
                                       with_dK=with_dK, workspace=workspace)
    else:
        out = H.fftconv_bwd(x.to(dev), al, be, H.kernel_spectrum(K), dy.to(dev), with_dK=with_dK,
                            workspace=workspace)
    torch.cuda.synchronize()
    return (x.float().numpy(), dy.float().numpy(), p, K.cpu().numpy(),
            [None if t is None else t.float().cpu().numpy() for t in out])


def _check(got, ref, dtype):
    assert all(np.all(np.isfinite(g)) for g in got)
    assert _rel(got[0], ref[0]) <= TOL_DX[dtype]
    for g, r in zip(got[1:], ref[1:]):
        assert g.shape == r.shape
        assert _rel(g, r) <= TOL_PARAM[dtype]


@pytest.mark.parametrize("n,B,C,dtype", [(2048, 2, 3, "f32"), (4096, 1, 2, "bf16"), (1 << 15, 3, 2, "f32"),
                                         (1 << 18, 1, 2, "bf16"), (1 << 20, 2, 1, "f32"), (1 << 22, 2, 1, "f32"),
                                         (1 << 23, 1, 1, "bf16"), (1 << 24, 1, 1, "f32")],
                         ids=lambda v: str(v))
def test_bwd_matches_fft_oracle(H, n, B, C, dtype):
    x, dy, p, K, got = _run_bwd(H, (n,), B, C, dtype, seed=300 + n % 89 + B)
    assert got[3].shape == (C, 2 * n - 1)
    _check(got, oracle.bwd_fft(x, p.alpha, p.beta, K, dy), dtype)


def test_bwd_sampled_gradients_match_direct_sums(H):
    n = 1 << 13
    x, dy, p, K, got = _run_bwd(H, (n,), 2, 2, "f32", seed=17)
    xp = synth.sample_points((n,), 2, 2, [(0, 0), (1, 1)], 16, seed=17)
    kp = synth.sample_kernel_points((n,), [0, 1], 16, seed=17)
    rx, rk = oracle.bwd_points(x, p.alpha, p.beta, K, dy, xp, kp)
    assert _rel(np.array([got[0][tuple(r)] for r in xp]), rx) <= 1e-4
    assert _rel(np.array([got[3][tuple(r)] for r in kp]), rk) <= 1e-4


def test_bwd_without_kernel_gradient_and_chunking(H):
    n, B, C = 1 << 12, 2, 5
    a = _run_bwd(H, (n,), B, C, "f32", seed=19)[4]
    b = _run_bwd(H, (n,), B, C, "f32", seed=19, with_dK=False)[4]
    assert b[3] is None
    for g, r in zip(b[:3], a[:3]):
        assert np.array_equal(g, r)
    minb = H.bwd_workspace_bytes(B, C, (n,), torch.float32, with_dK=True, minimum=True)
    for k in (1, 2):
        c = _run_bwd(H, (n,), B, C, "f32", seed=19, workspace=torch.empty(k * minb, dtype=torch.uint8, device="cuda"))[4]
        for g, r in zip(c, a):
            assert np.array_equal(g, r)


@pytest.mark.parametrize("n,B,C,dtype", [(1 << 14, 2, 2, "f32"), (1 << 22, 1, 1, "f32")], ids=lambda v: str(v))
def test_bwd_without_kernel_gradient_matches_fft_oracle(H, n, B, C, dtype):
    """Without dK the du rows take the row pass of their own (the correlation
    with the kernel spectrum): 2048- and 4096-point rows against the oracle."""
    x, dy, p, K, got = _run_bwd(H, (n,), B, C, dtype, seed=23 + n % 31, with_dK=False)
    assert got[3] is None
    ref = oracle.bwd_fft(x, p.alpha, p.beta, K, dy)
    _check(got[:3], ref[:3], dtype)


def test_bwd_per_sample_kernels(H):
    n = 1 << 13
    x, dy, p, Kb, got = _run_bwd(H, (n,), 3, 2, "f32", seed=21, per_sample=True)
    assert got[3].shape == (3, 2, 2 * n - 1)
    _check(got, oracle.bwd_fft_per_sample(x, p.alpha, p.beta, Kb, dy), "f32")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("idx", [5, 6])
def test_bwd_workload_full_size(H, idx):
    """The 2M- and 8M-token bf16 workloads at full size: the last channel's
    gradients against the FFT oracle."""
    wl = synth.WORKLOADS[idx]
    x, dy, p, K, got = _run_bwd(H, wl.dims, wl.B, wl.C, wl.dtype, seed=wl.seed)
    c = wl.C - 1
    ref = oracle.bwd_fft(x[:, c:c + 1], p.alpha[c:c + 1], p.beta[c:c + 1], K[c:c + 1], dy[:, c:c + 1])
    _check([got[0][:, c:c + 1], got[1][c:c + 1], got[2][c:c + 1], got[3][c:c + 1]], ref, wl.dtype)


def test_bwd_autograd_function(H):
    """gated_fftconv on a long 1-D signal: torch autograd through
    the library's forward and backward against the oracle's gradients."""
    n, B, C = 1 << 12, 2, 2
    dev = torch.device("cuda:0")
    p = synth.draw_params((n,), C, 23)
    x0 = synth.draw_x(p.rng, B, C, (n,), "f32")
    dy0 = synth.draw_dy((n,), B, C, "f32", 23)
    K0 = synth.kernel_channels((n,), p)
    x = x0.to(dev).requires_grad_()
    al = torch.from_numpy(p.alpha).to(dev).requires_grad_()
    be = torch.from_numpy(p.beta).to(dev).requires_grad_()
    K = K0.to(dev).requires_grad_()
    y = H.gated_fftconv(x, al, be, K)
    (y * dy0.to(dev)).sum().backward()
    ref = oracle.bwd_fft(x0.numpy(), p.alpha, p.beta, K0.numpy(), dy0.numpy())
    for t, r in zip((x.grad, al.grad, be.grad, K.grad), ref):
        assert _rel(t.cpu().numpy().astype(np.float64), r) <= 1e-4


def test_bwd_fused_du_rows_with_two_channels_per_chunk(H):
    """4096-point rows (n = 2^22, the kernel-gradient row kernel also writes the
    du rows) with two channels in one chunk, so its channel indexing (first
    channel of the chunk plus the row's channel) runs with more than one channel."""
    n, B, C = 1 << 22, 1, 2
    minb = H.bwd_workspace_bytes(B, C, (n,), torch.float32, with_dK=True, minimum=True)
    ws = torch.empty(2 * minb, dtype=torch.uint8, device="cuda")
    x, dy, p, K, got = _run_bwd(H, (n,), B, C, "f32", seed=29, workspace=ws)
    _check(got, oracle.bwd_fft(x, p.alpha, p.beta, K, dy), "f32")
