"""GPU parity of the circular mode (hyenand_fftconv_fwd_circ) against the fp64
CPU oracle's circular routes.

The circular mode is the gist.science summary's boundary handling for periodic
physical systems ("Methodology", "Boundary handling"): no padding, transforms
of length n, y[i] = sum_j phi(x[j]) x[j] K[(i-j) mod n].  Bar as for the
zero-padded forward: max|y_gpu - y_ref| / max|y_ref| <= 1e-4 (fp32 I/O),
<= 2e-2 (bf16 I/O).  Small grids against the direct sum, the seeded workloads
at full size against the unpadded FFT route on whole (b,c) slices.
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


def _inputs(dims, B, C, dtype, seed):
    p = synth.draw_params(dims, C, seed)
    x = synth.draw_x(p.rng, B, C, dims, dtype)
    K = synth.circular_kernel(dims, p)
    return x, p.alpha, p.beta, K


def _gpu(H, x, al, be, K, workspace=None):
    dev = torch.device("cuda:0")
    kh = H.kernel_spectrum_circ(K.to(dev))
    y = H.fftconv_fwd_circ(x.to(dev), torch.from_numpy(al).to(dev), torch.from_numpy(be).to(dev), kh,
                           workspace=workspace)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


SMALL = [((4,), 1, 1, "f32"), ((64,), 3, 3, "f32"), ((1024,), 2, 3, "f32"), ((256,), 1, 5, "bf16"),
         ((4, 4), 1, 1, "f32"), ((8, 4), 2, 3, "f32"), ((4, 16), 1, 2, "f32"), ((32, 32), 1, 4, "f32"),
         ((16, 64), 2, 2, "f32"), ((64, 16), 1, 3, "bf16"), ((4, 512), 1, 2, "f32"), ((512, 4), 1, 2, "f32"),
         ((4, 4, 4), 1, 1, "f32"), ((4, 8, 16), 2, 3, "f32"), ((16, 4, 8), 1, 2, "f32"), ((8, 16, 8), 2, 3, "bf16"),
         # maximum extents
         ((1024, 4), 1, 2, "f32"), ((4, 1024), 2, 1, "bf16"), ((1024, 4, 4), 1, 1, "f32"), ((4, 1024, 4), 1, 1, "f32"),
         ((4, 4, 1024), 1, 2, "f32")]


@pytest.mark.parametrize("dims,B,C,dtype", SMALL, ids=lambda v: str(v))
def test_small_grids_match_direct_sum(H, dims, B, C, dtype):
    x, al, be, K = _inputs(dims, B, C, dtype, seed=70 + sum(dims) + B + C)
    got = _gpu(H, x, al, be, K)
    ref = oracle.direct_circ(x.float().numpy(), al, be, K.numpy())
    assert np.all(np.isfinite(got))
    assert _rel(got, ref) <= TOL[dtype]


# (256, 4, 32): 256-point circular out-axis lines, row pairs fastest
@pytest.mark.parametrize("dims,B,C", [((128, 128), 2, 2), ((64, 256), 1, 2), ((32, 64, 16), 1, 2),
                                      ((1024, 1024), 1, 1), ((256, 4, 32), 2, 2)])
def test_medium_grids_match_fft_oracle(H, dims, B, C):
    x, al, be, K = _inputs(dims, B, C, "f32", seed=9)
    got = _gpu(H, x, al, be, K)
    ref = oracle.fftconv_circ(x.numpy(), al, be, K.numpy())
    assert _rel(got, ref) <= 1e-4


def test_shifted_delta_wraps(H):
    """A delta kernel at offset s rolls the gated input with wrap-around."""
    dims = (16, 32)
    x, al, be, _ = _inputs(dims, 1, 1, "f32", seed=4)
    K = torch.zeros((1,) + dims)
    K[0, 5, 30] = 1.0
    got = _gpu(H, x, al, be, K)[0, 0]
    u = oracle.gate(x[0, 0].numpy(), al[0], be[0])
    assert np.max(np.abs(got - np.roll(u, (5, 30), axis=(0, 1)))) <= 1e-5 * np.max(np.abs(u))


@pytest.mark.parametrize("dims,B,C,dtype", [((32, 32), 2, 7, "f32"), ((32, 32, 32), 1, 5, "bf16")],
                         ids=lambda v: str(v))
def test_every_chunking_gives_the_same_output(H, dims, B, C, dtype):
    x, al, be, K = _inputs(dims, B, C, dtype, seed=41)
    minb = H.circ_workspace_bytes(B, C, dims, x.dtype, minimum=True)
    outs = [_gpu(H, x, al, be, K, workspace=torch.empty(k * minb, dtype=torch.uint8, device="cuda"))
            for k in (1, 2, C)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def _full(H, wl, pairs):
    dev = torch.device("cuda:0")
    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x_t = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype)
    K = synth.circular_kernel(wl.dims, p, device=dev)
    kh = H.kernel_spectrum_circ(K)
    y = H.fftconv_fwd_circ(x_t.to(dev), torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev), kh)
    torch.cuda.synchronize()
    del kh
    K_h = K.cpu().numpy()
    del K
    y_h = y.float().cpu().numpy().reshape((wl.B * wl.C,) + wl.dims)
    assert np.all(np.isfinite(y_h))
    ref = oracle.fftconv_circ(x_t.float().numpy(), p.alpha, p.beta, K_h, pairs=pairs)
    return _rel(y_h[pairs], ref)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("idx,pairs", [(0, [0, 3]), (1, [0, 77, 511]), (2, [0, 255]), (3, [0, 31]), (4, [2])])
def test_workloads_full_size(H, idx, pairs):
    wl = synth.WORKLOADS[idx]
    assert _full(H, wl, pairs) <= TOL[wl.dtype]
