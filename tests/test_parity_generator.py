"""GPU parity of the input-dependent kernel generator (hyenand_generate_
kernel_spectrum: registers -> softmax control z(x) -> FiLM-modulated SIREN ->
Gaussian window, straight into the spectra) against the oracle's generator
(oracle.generate_kernels, spatial kernels in fp64) followed by the oracle's
DFT of each (b, c) kernel, and end to end through the per-sample forward
against the oracle's per-sample convolution.  Bars: spectra within 1e-4 of
their largest value (fp32 arithmetic, sincosf and 33-term sums on the GPU);
outputs max|d|/max|y| <= 1e-4 (fp32 I/O), 2e-2 (bf16 I/O)."""
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


def _case(dims, B, C, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, C) + tuple(dims)).astype(np.float32)
    x += (rng.uniform(-1, 1, (B, C)) * 2).astype(np.float32).reshape((B, C) + (1,) * len(dims))
    xt = torch.from_numpy(x)
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    gen = synth.draw_generator(dims, C, seed)
    a = rng.uniform(-1, 1, C).astype(np.float32)
    b = rng.uniform(-1, 1, C).astype(np.float32)
    return xt, gen, a, b


def _dev_gen(gen):
    return {k: (torch.from_numpy(v).cuda() if isinstance(v, np.ndarray) else v) for k, v in gen.items()}


def _layout_to_full(H, kh, dims, n):
    """Library layout of n spectra -> (main slots k_in >= 1 [n, No, Nm, S], Sv, Dv)."""
    d = len(dims)
    no, nm, ni = (1, 1, dims[0]) if d == 1 else ((dims[0], 1, dims[1]) if d == 2 else dims)
    No, Nm, S = (2 * no if d >= 2 else 1), (2 * nm if d == 3 else 1), ni
    T = H.spectrum_tile(dims)
    kh = kh.reshape(n, -1)
    main = kh[:, :No * Nm * S].reshape(n, S // T, No, Nm, T).transpose(0, 2, 3, 1, 4).reshape(n, No, Nm, S)
    dblk = kh[:, No * Nm * S:].reshape(n, No, Nm)
    return main, dblk, (No, Nm, 2 * ni)


@pytest.mark.parametrize("dims,B,C", [((64,), 2, 3), ((1024,), 1, 2), ((8, 16), 2, 3), ((64, 64), 2, 2),
                                      ((128, 32), 1, 3), ((8, 8, 8), 2, 2), ((16, 32, 8), 1, 2)],
                         ids=lambda v: str(v))
def test_spectra_match_the_oracle(H, dims, B, C):
    x, gen, _, _ = _case(dims, B, C, "f32", 50 + sum(dims))
    kh = H.generate_kernel_spectrum(x.cuda(), _dev_gen(gen)).cpu().numpy()
    K = oracle.generate_kernels(x.numpy(), gen)
    full = oracle.kernel_spectrum(K.reshape((B * C,) + K.shape[2:]).astype(np.float32), dims)
    main, dblk, (No, Nm, Ni) = _layout_to_full(H, kh, dims, B * C)
    full = full.reshape(B * C, No, Nm, Ni)
    S = Ni // 2
    g = 1.0 / (2 * No * Nm * Ni)
    scale = np.abs(full).max() * g
    assert np.abs(main[..., 1:] - g * full[..., 1:S]).max() <= 1e-4 * scale
    assert np.abs(main[..., 0] - g * (full[..., 0] + full[..., S]) / 2).max() <= 1e-4 * scale
    assert np.abs(dblk - g * (full[..., 0] - full[..., S]) / 2).max() <= 1e-4 * scale


@pytest.mark.parametrize("dims,B,C,dtype", [((256,), 3, 2, "f32"), ((32, 32), 2, 3, "f32"), ((16, 64), 2, 2, "bf16"),
                                            ((128, 128), 2, 2, "f32"), ((8, 16, 8), 2, 2, "f32")],
                         ids=lambda v: str(v))
def test_forward_with_generated_kernels(H, dims, B, C, dtype):
    x, gen, a, b = _case(dims, B, C, dtype, 90 + sum(dims))
    dev = torch.device("cuda:0")
    xd = x.to(dev)
    kh = H.generate_kernel_spectrum(xd, _dev_gen(gen))
    y = H.fftconv_fwd_per_sample(xd, torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev), kh)
    xf = x.float().numpy()
    K = oracle.generate_kernels(xf, gen).astype(np.float32)
    if int(np.prod(dims)) <= 4096:
        ref = oracle.direct_per_sample(xf, a, b, K)
    else:
        ref = oracle.fftconv_per_sample(xf, a, b, K)
    got = y.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - ref)) / np.max(np.abs(ref))) <= TOL[dtype]


def test_kernels_follow_the_input(H):
    """Samples with different statistics get different spectra; equal samples
    get bit-identical ones."""
    dims, B, C = (32, 32), 3, 2
    x, gen, _, _ = _case(dims, B, C, "f32", 7)
    x[2] = x[0]
    kh = H.generate_kernel_spectrum(x.cuda(), _dev_gen(gen)).reshape(B, C, -1)
    assert torch.equal(kh[2], kh[0])
    assert (kh[1] - kh[0]).abs().max() > 1e-3 * kh[0].abs().max()


@pytest.mark.parametrize("dims,B,C,dtype,chunked", [((256,), 3, 2, "f32", False), ((32, 32), 2, 3, "f32", False),
                                                    ((128, 64), 2, 5, "bf16", False), ((128, 64), 2, 5, "f32", True),
                                                    ((16, 32, 8), 2, 3, "f32", True),
                                                    ((64, 64, 64), 1, 4, "bf16", False)],
                         ids=lambda v: str(v))
def test_generated_forward_equals_generate_then_forward(H, dims, B, C, dtype, chunked):
    """hyenand_fftconv_fwd_generated gives the spectra and outputs of the two
    calls in sequence, bit for bit, also with the minimum workspace (every
    channel its own chunk)."""
    x, gen, a, b = _case(dims, B, C, dtype, 120 + sum(dims))
    dev = torch.device("cuda:0")
    xd, al, be, gd = x.to(dev), torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev), _dev_gen(gen)
    kh_ref = H.generate_kernel_spectrum(xd, gd)
    y_ref = H.fftconv_fwd_per_sample(xd, al, be, kh_ref)
    ws = None
    if chunked:
        ws = torch.empty(H.generated_workspace_bytes(B, C, dims, xd.dtype, minimum=True), dtype=torch.uint8,
                         device=dev)
    y, kh = H.fftconv_fwd_generated(xd, al, be, gd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(kh, kh_ref)
    assert torch.equal(y, y_ref)
    # Called again on another stream of the caller's, ordered after x is written there.
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x2 = (xd.float() * 0.5).to(xd.dtype)
        y2, kh2 = H.fftconv_fwd_generated(x2, al, be, gd, workspace=ws)
    s.synchronize()
    kh2_ref = H.generate_kernel_spectrum(x2, gd)
    assert torch.equal(kh2, kh2_ref)
    assert torch.equal(y2, H.fftconv_fwd_per_sample(x2, al, be, kh2_ref))


def test_generated_forward_in_a_graph(H):
    """The generated forward captured into a HIP graph and replayed with new
    inputs, eager work and synchronisations between the replays: every replay
    matches the eager calls."""
    dims, B, C = (64, 32), 2, 3
    x, gen, a, b = _case(dims, B, C, "f32", 140)
    dev = torch.device("cuda:0")
    xd, al, be, gd = x.to(dev), torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev), _dev_gen(gen)
    ws = torch.empty(H.generated_workspace_bytes(B, C, dims, xd.dtype), dtype=torch.uint8, device=dev)
    y = torch.empty_like(xd)
    kh = torch.empty(H.spectrum_bytes(B * C, dims) // 8, dtype=torch.complex64, device=dev).view(B * C, -1)
    H.fftconv_fwd_generated(xd, al, be, gd, K_hat=kh, y=y, workspace=ws)  # loads the kernels' code
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        H.fftconv_fwd_generated(xd, al, be, gd, K_hat=kh, y=y, workspace=ws)
    for k in range(3):
        xd.copy_(torch.from_numpy(x.numpy() * (1.0 + 0.25 * k) + 0.1 * k).to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        kh_ref = H.generate_kernel_spectrum(xd, gd)
        y_ref = H.fftconv_fwd_per_sample(xd, al, be, kh_ref)
        torch.cuda.synchronize()
        assert torch.equal(kh, kh_ref), f"replay {k}"
        assert torch.equal(y, y_ref), f"replay {k}"


@pytest.mark.parametrize("dims,B,C,R,D,dtype", [((2,), 1, 1, 1, 1, "f32"), ((4, 2), 2, 3, 64, 64, "f32"),
                                                ((2, 2, 2), 1, 2, 4, 8, "bf16"), ((1024,), 2, 3, 2, 3, "bf16"),
                                                ((16, 8, 32), 1, 5, 8, 2, "f32"), ((8, 64), 3, 1, 3, 5, "bf16")],
                         ids=lambda v: str(v))
def test_generator_extremes(H, dims, B, C, R, D, dtype):
    """The smallest grids (the VALU engine, S < 16), the largest register
    count and control width, single channels, odd channel counts and bf16
    inputs (the oracle reads the same bf16-rounded x)."""
    rng = np.random.default_rng(300 + sum(dims) + R)
    x = rng.standard_normal((B, C) + tuple(dims)).astype(np.float32)
    x += (rng.uniform(-1, 1, (B, C)) * 2).astype(np.float32).reshape((B, C) + (1,) * len(dims))
    xt = torch.from_numpy(x)
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    gen = synth.draw_generator(dims, C, 400 + R, R=R, D=D)
    kh = H.generate_kernel_spectrum(xt.cuda(), _dev_gen(gen)).cpu().numpy()
    K = oracle.generate_kernels(xt.float().numpy(), gen)
    full = oracle.kernel_spectrum(K.reshape((B * C,) + K.shape[2:]).astype(np.float32), dims)
    main, dblk, (No, Nm, Ni) = _layout_to_full(H, kh, dims, B * C)
    full = full.reshape(B * C, No, Nm, Ni)
    S = Ni // 2
    g = 1.0 / (2 * No * Nm * Ni)
    scale = np.abs(full).max() * g
    assert np.all(np.isfinite(kh))
    assert np.abs(main[..., 1:] - g * full[..., 1:S]).max() <= 1e-4 * scale
    assert np.abs(main[..., 0] - g * (full[..., 0] + full[..., S]) / 2).max() <= 1e-4 * scale
    assert np.abs(dblk - g * (full[..., 0] - full[..., S]) / 2).max() <= 1e-4 * scale
