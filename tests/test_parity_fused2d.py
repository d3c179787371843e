"""GPU parity of the on-chip 2-D forward (k_fused2d: one workgroup per (b, c)
pair, the half spectrum in LDS, one launch, no workspace) against the oracle's
direct sum, for every padded-length combination it takes (both extents in
[4, 64]), fp32 and bf16 I/O, shared and per-sample kernels.  The bar is the
parity tests' one: max|d|/max|y_ref| <= 1e-4 (fp32 I/O), <= 2e-2 (bf16 I/O)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
EXTENTS = (4, 8, 16, 32, 64)


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dimensional_fft_long_amd as H

    H.get_lib()
    return H


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


@pytest.mark.parametrize("n0", EXTENTS)
@pytest.mark.parametrize("n1", EXTENTS)
def test_every_extent_pair_matches_direct_sum(H, n0, n1):
    B, C = 2, 3
    dtype = "bf16" if (n0 * n1) % 3 == 1 else "f32"
    w = synth.make((n0, n1), B=B, C=C, dtype=dtype, seed=100 + n0 + 7 * n1)
    dev = torch.device("cuda:0")
    x = w["x"].to(dev)
    al, be = torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev)
    kh = H.kernel_spectrum(w["K"].to(dev))
    y = H.fftconv_fwd(x, al, be, kh)
    torch.cuda.synchronize()
    ref = oracle.direct(w["x"].float().numpy(), w["alpha"], w["beta"], w["K"].numpy())
    got = y.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert _rel(got, ref) <= TOL[dtype], (n0, n1, dtype)


@pytest.mark.parametrize("dims,B,C", [((64, 64), 3, 5), ((32, 64), 4, 9), ((64, 8), 1, 17)])
def test_batches_and_channels(H, dims, B, C):
    """More (b, c) pairs than 8 and a pair count that is not a multiple of 8
    (the XCD-blocked pair order keeps a plain tail)."""
    w = synth.make(dims, B=B, C=C, dtype="f32", seed=7 + B + C)
    dev = torch.device("cuda:0")
    kh = H.kernel_spectrum(w["K"].to(dev))
    y = H.fftconv_fwd(w["x"].to(dev), torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev), kh)
    ref = oracle.fftconv(w["x"].numpy(), w["alpha"], w["beta"], w["K"].numpy())
    assert _rel(y.cpu().numpy(), ref) <= 1e-4


def test_per_sample_kernels(H):
    dims, B, C = (64, 32), 3, 2
    dev = torch.device("cuda:0")
    p = synth.draw_params(dims, C, 33)
    x = synth.draw_x(p.rng, B, C, dims, "f32")
    K = synth.kernel_channels(dims, p)
    Kb = torch.stack([K * (0.5 + 0.25 * b) for b in range(B)])
    kh = H.kernel_spectrum_per_sample(Kb.to(dev))
    y = H.fftconv_fwd_per_sample(x.to(dev), torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev), kh)
    ref = oracle.direct_per_sample(x.numpy(), p.alpha, p.beta, Kb.numpy())
    assert _rel(y.cpu().numpy(), ref) <= 1e-4


def test_shifted_delta_every_output(H):
    """K = delta_s, mixed-sign shift: y[i] = u[i - s] inside the shifted box and
    0 elsewhere (the zero-padded boundary), at the largest fused grid."""
    dims, B, C, s = (64, 64), 2, 3, (-25, 37)
    dev = torch.device("cuda:0")
    p = synth.draw_params(dims, C, 41)
    x = synth.draw_x(p.rng, B, C, dims, "f32")
    K = torch.zeros((C, 127, 127))
    K[:, 63 + s[0], 63 + s[1]] = 1.0
    y = H.fftconv_fwd(x.to(dev), torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev),
                      H.kernel_spectrum(K.to(dev))).cpu().numpy()
    for b in range(B):
        for c in range(C):
            u = oracle.gate(x[b, c].numpy(), float(p.alpha[c]), float(p.beta[c]))
            exp = np.zeros(dims)
            exp[0:64 + s[0], s[1]:64] = u[-s[0]:64, 0:64 - s[1]]
            assert np.max(np.abs(y[b, c] - exp)) <= 1e-5 * np.max(np.abs(u))


def test_workload_2d_128_three_pass(H):
    """128^2 (above the on-chip limit: the three-pass path) with the 256^2
    image's batch and channels, whole pairs against the FFT oracle."""
    wl = {w.name: w for w in synth.WORKLOADS}["2d_128x128_b8_c64_f32"]
    dev = torch.device("cuda:0")
    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype)
    K = synth.kernel_channels(wl.dims, p)
    y = H.fftconv_fwd(x.to(dev), torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev),
                      H.kernel_spectrum(K.to(dev))).cpu().numpy()
    P = wl.B * wl.C
    pairs = [0, 77, 300, P - 1]
    ref = oracle.fftconv(x.numpy(), p.alpha, p.beta, K.numpy(), pairs=pairs)
    assert _rel(y.reshape((P,) + wl.dims)[pairs], ref) <= 1e-4
