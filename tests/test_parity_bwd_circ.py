"""GPU parity of the circular-mode backward (hyenand_fftconv_bwd_circ) against
the fp64 CPU oracle's circular backward routes.

The circular mode is the gist.science summary's boundary handling for periodic
physical systems ("Methodology", "Boundary handling"): y[i] = sum_j u[j]
K[(i-j) mod n].  Its backward takes every offset modulo n:
du[j] = sum_i dy[i] K[(i-j) mod n], dK[m] = sum_b sum_j dy[(j+m) mod n] u[j],
dx = du (s + alpha x s (1-s)).  Bar as for the zero-padded backward:
max|g_gpu - g_ref| / max|g_ref| <= 1e-4 for fp32 I/O; bf16 I/O: dx <= 2e-2,
dalpha, dbeta, dK (fp32 outputs) <= 1e-3.  Small grids against the direct
sums, the seeded workloads at full size on whole channels through the
unpadded FFT route.
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


def _inputs(dims, B, C, dtype, seed):
    p = synth.draw_params(dims, C, seed)
    x = synth.draw_x(p.rng, B, C, dims, dtype)
    K = synth.circular_kernel(dims, p)
    dy = synth.draw_dy(dims, B, C, dtype, seed)
    return x, p.alpha, p.beta, K, dy


def _gpu_bwd(H, x, al, be, K, dy, with_dK=True, workspace=None):
    dev = torch.device("cuda:0")
    kh = H.kernel_spectrum_circ(K.to(dev))
    out = H.fftconv_bwd_circ(x.to(dev), torch.from_numpy(al).to(dev), torch.from_numpy(be).to(dev), kh,
                             dy.to(dev), with_dK=with_dK, workspace=workspace)
    torch.cuda.synchronize()
    return [None if t is None else t.float().cpu().numpy() for t in out]


SMALL = [((4,), 1, 1, "f32"), ((64,), 3, 3, "f32"), ((1024,), 2, 3, "f32"), ((256,), 2, 5, "bf16"),
         ((4, 4), 1, 1, "f32"), ((8, 4), 2, 3, "f32"), ((4, 16), 3, 2, "f32"), ((32, 32), 2, 4, "f32"),
         ((16, 64), 2, 2, "f32"), ((64, 16), 1, 3, "bf16"), ((4, 512), 1, 2, "f32"), ((512, 4), 2, 2, "f32"),
         ((4, 4, 4), 1, 1, "f32"), ((4, 8, 16), 2, 3, "f32"), ((16, 4, 8), 1, 2, "f32"), ((8, 8, 8), 3, 1, "f32"),
         ((8, 16, 8), 2, 3, "bf16"),
         # maximum extents
         ((1024, 4), 2, 2, "f32"), ((4, 1024), 1, 3, "bf16"), ((1024, 4, 4), 1, 2, "f32"),
         ((4, 1024, 4), 2, 1, "f32"), ((4, 4, 1024), 1, 2, "bf16")]


@pytest.mark.parametrize("dims,B,C,dtype", SMALL, ids=lambda v: str(v))
def test_small_grids_match_direct_sums(H, dims, B, C, dtype):
    x, al, be, K, dy = _inputs(dims, B, C, dtype, seed=90 + sum(dims) + B + C)
    got = _gpu_bwd(H, x, al, be, K, dy)
    ref = oracle.bwd_direct_circ(x.float().numpy(), al, be, K.numpy(), dy.float().numpy())
    assert all(np.all(np.isfinite(g)) for g in got)
    assert got[3].shape == (C,) + dims
    assert _rel(got[0], ref[0]) <= TOL_DX[dtype]
    for g, r in zip(got[1:], ref[1:]):
        assert _rel(g, r) <= TOL_PARAM[dtype]


# (256, 4, 32): 256-point circular out-axis lines, the backward's 8-slot tiles
# of 16-slot runs in the work-item order
@pytest.mark.parametrize("dims,B,C", [((128, 128), 2, 2), ((64, 256), 3, 2), ((32, 64, 16), 2, 2),
                                      ((1024,), 3, 2), ((256, 4, 32), 2, 2)])
def test_medium_grids_match_fft_oracle(H, dims, B, C):
    x, al, be, K, dy = _inputs(dims, B, C, "f32", seed=12)
    got = _gpu_bwd(H, x, al, be, K, dy)
    ref = oracle.bwd_fft_circ(x.numpy(), al, be, K.numpy(), dy.numpy())
    for g, r in zip(got, ref):
        assert _rel(g, r) <= 1e-4


def test_shifted_delta_rolls_the_gradient_back(H):
    """A delta kernel at offset s: du is dy rolled by -s with wrap-around."""
    dims = (16, 32)
    x, al, be, _, dy = _inputs(dims, 1, 1, "f32", seed=5)
    K = torch.zeros((1,) + dims)
    K[0, 5, 30] = 1.0
    dx = _gpu_bwd(H, x, al, be, K, dy, with_dK=False)[0][0, 0]
    xs = x[0, 0].numpy().astype(np.float64)
    s = 1.0 / (1.0 + np.exp(-(float(al[0]) * xs + float(be[0]))))
    want = np.roll(dy[0, 0].numpy().astype(np.float64), (-5, -30), axis=(0, 1)) * (s + float(al[0]) * xs * s * (1 - s))
    assert _rel(dx, want) <= 1e-5


def test_without_kernel_gradient(H):
    """dK = NULL: same dx, dalpha, dbeta, bit for bit, with the smaller workspace."""
    for dims in [(32, 16), (8, 4, 16), (128,)]:
        x, al, be, K, dy = _inputs(dims, 2, 3, "f32", seed=13)
        a = _gpu_bwd(H, x, al, be, K, dy, with_dK=True)
        b = _gpu_bwd(H, x, al, be, K, dy, with_dK=False)
        assert b[3] is None
        for g, r in zip(b[:3], a[:3]):
            assert np.array_equal(g, r)


@pytest.mark.parametrize("dims,B,C,dtype", [((32, 32), 2, 7, "f32"), ((16, 16, 16), 1, 5, "bf16"),
                                            ((64,), 3, 5, "f32")], ids=lambda v: str(v))
def test_every_chunking_gives_the_same_gradients(H, dims, B, C, dtype):
    x, al, be, K, dy = _inputs(dims, B, C, dtype, seed=60 + C)
    minb = H.bwd_workspace_bytes(B, C, dims, x.dtype, with_dK=True, minimum=True, circular=True)
    outs = [_gpu_bwd(H, x, al, be, K, dy, workspace=torch.empty(k * minb, dtype=torch.uint8, device="cuda"))
            for k in (1, 2, C)]
    for o in outs[1:]:
        for g, r in zip(o, outs[0]):
            if len(dims) == 1:
                assert _rel(g, r) <= 1e-6  # 1-D pairing follows the chunk boundaries
            else:
                assert np.array_equal(g, r)


def test_autograd_function(H):
    """gated_fftconv with circular=True: torch autograd through the
    library's circular forward and backward against the oracle's gradients."""
    dims, B, C = (16, 8), 2, 3
    x0, al0, be0, K0, dy0 = _inputs(dims, B, C, "f32", seed=14)
    x = x0.cuda().requires_grad_()
    al = torch.from_numpy(al0).cuda().requires_grad_()
    be = torch.from_numpy(be0).cuda().requires_grad_()
    K = K0.cuda().requires_grad_()
    y = H.gated_fftconv(x, al, be, K, True)
    (y * dy0.cuda()).sum().backward()
    ref = oracle.bwd_direct_circ(x0.numpy(), al0, be0, K0.numpy(), dy0.numpy())
    for t, r in zip((x.grad, al.grad, be.grad, K.grad), ref):
        assert _rel(t.cpu().numpy(), r) <= 1e-4


def test_workspace_too_small_is_rejected(H):
    dims, B, C = (32, 32), 1, 2
    x, al, be, K, dy = _inputs(dims, B, C, "f32", seed=3)
    minb = H.bwd_workspace_bytes(B, C, dims, x.dtype, with_dK=True, minimum=True, circular=True)
    with pytest.raises(H.HyenandError):
        _gpu_bwd(H, x, al, be, K, dy, workspace=torch.empty(minb - 8, dtype=torch.uint8, device="cuda"))


def _full(H, wl, chans):
    dev = torch.device("cuda:0")
    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x_t = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype)
    dy_t = synth.draw_dy(wl.dims, wl.B, wl.C, wl.dtype, wl.seed)
    K = synth.circular_kernel(wl.dims, p, device=dev)
    kh = H.kernel_spectrum_circ(K)
    dx, da, db, dK = H.fftconv_bwd_circ(x_t.to(dev), torch.from_numpy(p.alpha).to(dev),
                                        torch.from_numpy(p.beta).to(dev), kh, dy_t.to(dev))
    torch.cuda.synchronize()
    del kh
    K_h = K.cpu().numpy()
    del K
    dx_h = dx[:, chans].float().cpu().numpy()
    del dx
    da_h, db_h, dK_h = da.cpu().numpy()[chans], db.cpu().numpy()[chans], dK[chans].cpu().numpy()
    del dK
    assert np.all(np.isfinite(dx_h)) and np.all(np.isfinite(dK_h))
    r = oracle.bwd_fft_circ(x_t.float().numpy(), p.alpha, p.beta, K_h, dy_t.float().numpy(), chans=chans)
    return {"dx": _rel(dx_h, r[0]), "da": _rel(da_h, r[1]), "db": _rel(db_h, r[2]), "dK": _rel(dK_h, r[3])}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("idx,chans", [(0, [0, 3]), (1, [0, 63]), (2, [127]), (3, [31]), (4, [2])])
def test_workloads_full_size(H, idx, chans):
    wl = synth.WORKLOADS[idx]
    errs = _full(H, wl, chans)
    for k, v in errs.items():
        assert v <= (TOL_DX if k == "dx" else TOL_PARAM)[wl.dtype], (k, v, errs)
