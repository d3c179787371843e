"""GPU parity of the forward with input-dependent kernels
(hyenand_fftconv_fwd_per_sample): one kernel per (b, c), as the gist.science
summary's kernels conditioned on the whole input sample ("Input dependent
kernels via registers and FiLM", "Kernel synthesis").  Against the oracle's
per-sample routes; bar as for the shared-kernel forward (1e-4 fp32, 2e-2 bf16).
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


def _inputs(dims, B, C, dtype, seed, device="cpu"):
    """Per-sample kernels: the synthetic generator's kernel of each channel,
    scaled and shifted by a seeded per-(b, c) factor (a stand-in for the
    summary's FiLM modulation), so that every batch entry differs."""
    p = synth.draw_params(dims, C, seed)
    x = synth.draw_x(p.rng, B, C, dims, dtype)
    K = synth.kernel_channels(dims, p, device=device)
    rng = np.random.Generator(np.random.PCG64([seed, 3]))
    g = torch.from_numpy(rng.uniform(0.5, 1.5, (B, C)).astype(np.float32)).to(K.device)
    h = torch.from_numpy(rng.uniform(-0.1, 0.1, (B, C)).astype(np.float32)).to(K.device)
    shape = (B, C) + (1,) * len(dims)
    Kb = (K.unsqueeze(0) * g.reshape(shape) + h.reshape(shape)).contiguous()
    return x, p.alpha, p.beta, Kb


def _gpu(H, x, al, be, Kb):
    dev = torch.device("cuda:0")
    kh = H.kernel_spectrum_per_sample(Kb.to(dev))
    y = H.fftconv_fwd_per_sample(x.to(dev), torch.from_numpy(al).to(dev), torch.from_numpy(be).to(dev), kh)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


@pytest.mark.parametrize("dims,B,C,dtype", [((64,), 3, 3, "f32"), ((256,), 2, 5, "bf16"), ((8, 4), 2, 3, "f32"),
                                            ((32, 32), 3, 4, "f32"), ((64, 16), 2, 3, "bf16"),
                                            ((4, 8, 16), 2, 3, "f32"), ((8, 16, 8), 3, 2, "bf16")],
                         ids=lambda v: str(v))
def test_small_grids_match_direct_sum(H, dims, B, C, dtype):
    x, al, be, Kb = _inputs(dims, B, C, dtype, seed=90 + sum(dims))
    got = _gpu(H, x, al, be, Kb)
    ref = oracle.direct_per_sample(x.float().numpy(), al, be, Kb.numpy())
    assert _rel(got, ref) <= TOL[dtype]


def test_equal_kernels_match_the_shared_spectrum(H):
    dims, B, C = (64, 64), 3, 4
    p = synth.draw_params(dims, C, 5)
    x = synth.draw_x(p.rng, B, C, dims, "f32").cuda()
    K = synth.kernel_channels(dims, p).cuda()
    al, be = torch.from_numpy(p.alpha).cuda(), torch.from_numpy(p.beta).cuda()
    y_shared = H.fftconv_fwd(x, al, be, H.kernel_spectrum(K))
    y_ps = H.fftconv_fwd_per_sample(x, al, be, H.kernel_spectrum_per_sample(K.unsqueeze(0).repeat(B, 1, 1, 1)))
    torch.cuda.synchronize()
    assert torch.equal(y_shared, y_ps)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("idx,cases", [(1, [(0, 3), (7, 60)]), (2, [(1, 100)]), (3, [(0, 17)])])
def test_workloads_full_size(H, idx, cases):
    """Full size; whole (b, c) slices against the FFT oracle with that pair's own kernel."""
    wl = synth.WORKLOADS[idx]
    x, al, be, Kb = _inputs(wl.dims, wl.B, wl.C, wl.dtype, seed=wl.seed, device="cuda")
    got = _gpu(H, x, al, be, Kb)
    xf = x.float().numpy()
    for b, c in cases:
        ref = oracle.fftconv(xf[b:b + 1, c:c + 1], al[c:c + 1], be[c:c + 1], Kb[b, c:c + 1].cpu().numpy())
        assert _rel(got[b, c], ref[0, 0]) <= TOL[wl.dtype], (b, c)
