"""GPU parity of the backward with input-dependent kernels
(hyenand_fftconv_bwd_per_sample) against the fp64 CPU oracle's per-sample
backward routes.

The kernels are conditioned on the whole input sample (gist.science summary,
"Input dependent kernels via registers and FiLM", "Kernel synthesis"), so the
kernel gradient is one dK per (b, c), which is what flows back into a kernel
generator; alpha and beta are shared by the samples and their gradients sum
over the batch.  Bar as for the shared-kernel backward: max|g - g_ref| /
max|g_ref| <= 1e-4 for fp32 I/O; bf16 I/O: dx <= 2e-2, dalpha, dbeta,
dK <= 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL_DX = {"f32": 1e-4, "bf16": 2e-2}
TOL_PARAM = {"f32": 1e-4, "bf16": 1e-3}


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dimensional_fft_long_amd as H

    H.get_lib()
    return H


def _rel(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def _inputs(dims, B, C, dtype, seed, device="cpu"):
    """Per-sample kernels: each channel's synthetic kernel scaled and shifted by
    a seeded per-(b, c) factor, so that every batch entry differs."""
    p = synth.draw_params(dims, C, seed)
    x = synth.draw_x(p.rng, B, C, dims, dtype)
    K = synth.kernel_channels(dims, p, device=device)
    rng = np.random.Generator(np.random.PCG64([seed, 3]))
    g = torch.from_numpy(rng.uniform(0.5, 1.5, (B, C)).astype(np.float32)).to(K.device)
    h = torch.from_numpy(rng.uniform(-0.1, 0.1, (B, C)).astype(np.float32)).to(K.device)
    shape = (B, C) + (1,) * len(dims)
    Kb = (K.unsqueeze(0) * g.reshape(shape) + h.reshape(shape)).contiguous()
    dy = synth.draw_dy(dims, B, C, dtype, seed)
    return x, p.alpha, p.beta, Kb, dy


def _gpu_bwd(H, x, al, be, Kb, dy, with_dK=True, workspace=None):
    dev = torch.device("cuda:0")
    kh = H.kernel_spectrum_per_sample(Kb.to(dev))
    out = H.fftconv_bwd_per_sample(x.to(dev), torch.from_numpy(al).to(dev), torch.from_numpy(be).to(dev), kh,
                                   dy.to(dev), with_dK=with_dK, workspace=workspace)
    torch.cuda.synchronize()
    return [None if t is None else t.float().cpu().numpy() for t in out]


SMALL = [((64,), 3, 3, "f32"), ((1024,), 2, 2, "f32"), ((256,), 2, 5, "bf16"), ((8, 4), 2, 3, "f32"),
         ((32, 32), 3, 4, "f32"), ((64, 16), 2, 3, "bf16"), ((2, 512), 2, 2, "f32"), ((4, 8, 16), 2, 3, "f32"),
         ((8, 16, 8), 3, 2, "bf16"), ((2, 2, 64), 2, 2, "f32")]


@pytest.mark.parametrize("dims,B,C,dtype", SMALL, ids=lambda v: str(v))
def test_small_grids_match_direct_sums(H, dims, B, C, dtype):
    x, al, be, Kb, dy = _inputs(dims, B, C, dtype, seed=120 + sum(dims) + B)
    got = _gpu_bwd(H, x, al, be, Kb, dy)
    ref = oracle.bwd_direct_per_sample(x.float().numpy(), al, be, Kb.numpy(), dy.float().numpy())
    assert all(np.all(np.isfinite(g)) for g in got)
    assert got[3].shape == (B, C) + tuple(2 * n - 1 for n in dims)
    assert _rel(got[0], ref[0]) <= TOL_DX[dtype]
    for g, r in zip(got[1:], ref[1:]):
        assert _rel(g, r) <= TOL_PARAM[dtype]


def test_equal_kernels_match_the_shared_backward(H):
    """The same kernel for every sample: dx equals the shared-kernel backward's,
    dalpha / dbeta agree to fp32 rounding (summed per sample, then over the
    batch) and dK summed over the batch is the shared dK."""
    dims, B, C = (64, 32), 3, 4
    p = synth.draw_params(dims, C, 7)
    x = synth.draw_x(p.rng, B, C, dims, "f32").cuda()
    dy = synth.draw_dy(dims, B, C, "f32", 7).cuda()
    K = synth.kernel_channels(dims, p).cuda()
    al, be = torch.from_numpy(p.alpha).cuda(), torch.from_numpy(p.beta).cuda()
    sh = H.fftconv_bwd(x, al, be, H.kernel_spectrum(K), dy)
    ps = H.fftconv_bwd_per_sample(x, al, be, H.kernel_spectrum_per_sample(K.unsqueeze(0).repeat(B, 1, 1, 1)), dy)
    torch.cuda.synchronize()
    assert torch.equal(sh[0], ps[0])
    for i in (1, 2):
        assert _rel(ps[i].cpu().numpy(), sh[i].cpu().numpy().astype(np.float64)) <= 1e-5
    assert _rel(ps[3].sum(0).cpu().numpy(), sh[3].cpu().numpy().astype(np.float64)) <= 1e-5


def test_without_kernel_gradient_and_chunking(H):
    dims, B, C = (32, 16), 2, 5
    x, al, be, Kb, dy = _inputs(dims, B, C, "f32", seed=9)
    a = _gpu_bwd(H, x, al, be, Kb, dy)
    b = _gpu_bwd(H, x, al, be, Kb, dy, with_dK=False)
    assert b[3] is None
    for g, r in zip(b[:3], a[:3]):
        assert np.array_equal(g, r)
    minb = H.bwd_workspace_bytes(1, C, dims, torch.float32, with_dK=True, minimum=True)
    for k in (1, 2):
        c = _gpu_bwd(H, x, al, be, Kb, dy, workspace=torch.empty(k * minb, dtype=torch.uint8, device="cuda"))
        for g, r in zip(c, a):
            assert np.array_equal(g, r)
    with pytest.raises(H.HyenandError):
        _gpu_bwd(H, x, al, be, Kb, dy, workspace=torch.empty(minb - 8, dtype=torch.uint8, device="cuda"))


def test_autograd_function(H):
    """gated_fftconv with kernels [B, C, ...]: torch autograd through
    the per-sample forward and backward against the oracle's gradients."""
    dims, B, C = (16, 8), 3, 2
    x0, al0, be0, K0, dy0 = _inputs(dims, B, C, "f32", seed=15)
    x = x0.cuda().requires_grad_()
    al = torch.from_numpy(al0).cuda().requires_grad_()
    be = torch.from_numpy(be0).cuda().requires_grad_()
    K = K0.cuda().requires_grad_()
    y = H.gated_fftconv(x, al, be, K)
    (y * dy0.cuda()).sum().backward()
    ref = oracle.bwd_direct_per_sample(x0.numpy(), al0, be0, K0.numpy(), dy0.numpy())
    for t, r in zip((x.grad, al.grad, be.grad, K.grad), ref):
        assert t.shape == r.shape
        assert _rel(t.cpu().numpy(), r) <= 1e-4


@pytest.mark.timeout(600)
@pytest.mark.parametrize("idx,chan,pairs", [(1, 5, [(0, 5), (7, 60)]), (2, 100, [(1, 100)]), (3, 17, [(0, 17)])])
def test_workloads_full_size(H, idx, chan, pairs):
    """Full size; whole (b, c) slices of dx and dK against the FFT oracle with
    that pair's own kernel, and dalpha / dbeta of one channel summed over its
    batch entries."""
    wl = synth.WORKLOADS[idx]
    x, al, be, Kb, dy = _inputs(wl.dims, wl.B, wl.C, wl.dtype, seed=wl.seed, device="cuda")
    dev = torch.device("cuda:0")
    kh = H.kernel_spectrum_per_sample(Kb)
    dx, da, db, dK = H.fftconv_bwd_per_sample(x.to(dev), torch.from_numpy(al).to(dev), torch.from_numpy(be).to(dev),
                                              kh, dy.to(dev))
    torch.cuda.synchronize()
    del kh
    xf, dyf = x.float().numpy(), dy.float().numpy()
    errs = {}
    for b, c in pairs:
        r = oracle.bwd_fft(xf[b:b + 1, c:c + 1], al[c:c + 1], be[c:c + 1], Kb[b, c:c + 1].cpu().numpy(),
                           dyf[b:b + 1, c:c + 1])
        errs[f"dx{b},{c}"] = _rel(dx[b, c].float().cpu().numpy(), r[0][0, 0])
        errs[f"dK{b},{c}"] = _rel(dK[b, c].cpu().numpy(), r[3][0])
    sa = sb = 0.0
    for b in range(wl.B):
        r = oracle.bwd_fft(xf[b:b + 1, chan:chan + 1], al[chan:chan + 1], be[chan:chan + 1],
                           Kb[b, chan:chan + 1].cpu().numpy(), dyf[b:b + 1, chan:chan + 1])
        sa += float(r[1][0])
        sb += float(r[2][0])
    scale = max(abs(sa), abs(sb))
    errs["da"] = abs(float(da[chan]) - sa) / scale
    errs["db"] = abs(float(db[chan]) - sb) / scale
    for k, v in errs.items():
        assert v <= (TOL_DX if k.startswith("dx") else TOL_PARAM)[wl.dtype], (k, v, errs)
