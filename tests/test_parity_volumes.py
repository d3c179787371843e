"""GPU parity of the largest volumes at full size, in the launch configuration
the benchmark uses (the library's recommended workspace).

* Sampled outputs of every (b, c) pair against the oracle's direct sums: the
  corners, the centre, every edge midpoint and face centre of the grid box, and
  64 seeded random voxels per pair.
* A shifted delta kernel K = delta_s with a mixed-sign shift on every axis:
  then y[i] = u[i - s] where i - s lies in the grid and 0 elsewhere (the output
  equation of the explainer "Native multi-dimensional subquadratic operators
  via input-dependent long convolutions", section "HyenaND: native-space
  implicit global kernel", with the zero-padded, non-circular boundary of the
  gist.science summary, "Methodology", "Boundary handling"), so EVERY voxel of
  y is compared against the oracle's gate u = phi(x) x moved by s: every store,
  index and crop of the real plan is exercised.
* The backward with the same delta kernel: du[j] = dy[j + s] (zero where
  j + s leaves the grid), so dx at every voxel and dalpha, dbeta exactly follow
  from the oracle's gate derivative (oracle.gate_vjp) on the shifted dy; dK at
  sampled offsets against the oracle's direct sums.

Bars as everywhere: max|d| / max|ref| <= 1e-4 (fp32 I/O) or 2e-2 (bf16 I/O);
dalpha, dbeta and dK are fp32 outputs (1e-4 / 1e-3 as in the backward tests).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL_PARAM = {"f32": 1e-4, "bf16": 1e-3}
BIG = {"3d_512x512x512_b1_c4_bf16": (37, -101, 5), "3d_1024x1024x256_b1_c2_f32": (-300, 17, -64),
       "3d_512x512x64_b1_c16_f32": (-5, 250, -31)}


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dimensional_fft_long_amd as H

    H.get_lib()
    return H


def _wl(name):
    return {w.name: w for w in synth.WORKLOADS}[name]


def _shift_slices(dims, s):
    """(destination, source) slices with dst = src + s inside the grid."""
    dst = tuple(slice(max(0, k), n + min(0, k)) for n, k in zip(dims, s))
    src = tuple(slice(max(0, -k), n - max(0, k)) for n, k in zip(dims, s))
    return dst, src


def _delta_kernel(wl, s, dev):
    K = torch.zeros((wl.C,) + tuple(2 * n - 1 for n in wl.dims), dtype=torch.float32, device=dev)
    K[(slice(None),) + tuple(n - 1 + k for n, k in zip(wl.dims, s))] = 1.0
    return K


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["3d_512x512x512_b1_c4_bf16", "3d_1024x1024x256_b1_c2_f32"])
def test_sampled_every_pair(H, name):
    wl = _wl(name)
    print(f"[sampled] {name}", flush=True)
    dev = torch.device("cuda:0")
    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x_t = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype)
    K = synth.kernel_channels(wl.dims, p, device=dev)
    kh = H.kernel_spectrum(K)
    y = H.fftconv_fwd(x_t.to(dev), torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev), kh)
    torch.cuda.synchronize()
    del kh
    K_h = K.cpu().numpy()
    del K
    y_h = y.float().cpu().numpy()
    del y
    assert np.all(np.isfinite(y_h))
    pairs = [(b, c) for b in range(wl.B) for c in range(wl.C)][:4]
    pts = synth.sample_points(wl.dims, wl.B, wl.C, pairs, 64, seed=wl.seed + 7, edges=True)
    assert len(pts) == len(pairs) * (8 + 1 + 12 + 6 + 64)
    ref = oracle.direct_points(x_t.float().numpy(), p.alpha, p.beta, K_h, pts)
    got = np.array([y_h[tuple(r)] for r in pts])
    err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    print(f"[sampled] {name}: {len(pts)} points, rel err {err:.3e}", flush=True)
    assert err <= TOL[wl.dtype]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(BIG))
def test_shifted_delta_every_voxel(H, name):
    wl = _wl(name)
    s = BIG[name]
    print(f"[delta] {name} shift {s}", flush=True)
    dev = torch.device("cuda:0")
    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x_t = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype)
    K = _delta_kernel(wl, s, dev)
    kh = H.kernel_spectrum(K)
    del K
    y = H.fftconv_fwd(x_t.to(dev), torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev), kh)
    torch.cuda.synchronize()
    del kh
    dst, src = _shift_slices(wl.dims, s)
    x_h = x_t.float().numpy()
    worst = 0.0
    for b in range(wl.B):
        for c in range(wl.C):
            u = oracle.gate(x_h[b, c], float(p.alpha[c]), float(p.beta[c]))
            exp = np.zeros(wl.dims, dtype=np.float64)
            exp[dst] = u[src]
            got = y[b, c].float().cpu().numpy()
            scale = float(np.max(np.abs(u)))
            err = float(np.max(np.abs(got - exp))) / scale
            outside = got.copy()
            outside[dst] = 0.0
            print(f"[delta] {name} pair ({b},{c}): rel err {err:.3e}, max outside the shifted box "
                  f"{float(np.max(np.abs(outside))) / scale:.3e}", flush=True)
            worst = max(worst, err)
    assert worst <= TOL[wl.dtype]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["3d_512x512x512_b1_c4_bf16", "3d_1024x1024x256_b1_c2_f32"])
def test_backward_shifted_delta_every_voxel(H, name):
    wl = _wl(name)
    s = BIG[name]
    print(f"[delta bwd] {name} shift {s}", flush=True)
    dev = torch.device("cuda:0")
    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x_t = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype)
    dy_t = synth.draw_dy(wl.dims, wl.B, wl.C, wl.dtype, wl.seed)
    K = _delta_kernel(wl, s, dev)
    kh = H.kernel_spectrum(K)
    del K
    dx, da, db, dK = H.fftconv_bwd(x_t.to(dev), torch.from_numpy(p.alpha).to(dev),
                                   torch.from_numpy(p.beta).to(dev), kh, dy_t.to(dev))
    torch.cuda.synchronize()
    del kh
    da_h, db_h = da.cpu().numpy().astype(np.float64), db.cpu().numpy().astype(np.float64)
    x_h, dy_h = x_t.float().numpy(), dy_t.float().numpy()
    # du[j] = sum_i dy[i] K[i - j] = dy[j + s]: the source box of the forward is
    # where j + s stays inside the grid.
    dst, src = _shift_slices(wl.dims, s)
    errs = {}
    ref_a = np.zeros(wl.C)
    ref_b = np.zeros(wl.C)
    for c in range(wl.C):
        for b in range(wl.B):
            du = np.zeros(wl.dims, dtype=np.float64)
            du[src] = dy_h[b, c][dst]
            ref_dx, sa, sb = oracle.gate_vjp(x_h[b, c], du, float(p.alpha[c]), float(p.beta[c]))
            ref_a[c] += sa
            ref_b[c] += sb
            got = dx[b, c].float().cpu().numpy()
            errs[f"dx({b},{c})"] = float(np.max(np.abs(got - ref_dx)) / np.max(np.abs(ref_dx)))
    errs["dalpha"] = float(np.max(np.abs(da_h - ref_a)) / np.max(np.abs(ref_a)))
    errs["dbeta"] = float(np.max(np.abs(db_h - ref_b)) / np.max(np.abs(ref_b)))
    # dK at sampled offsets (every corner, offset 0, the shift itself, random)
    kp = synth.sample_kernel_points(wl.dims, list(range(min(wl.C, 2))), 6, seed=wl.seed)
    kp = np.concatenate([kp, np.array([[0] + [n - 1 + k for n, k in zip(wl.dims, s)]], dtype=np.int64)])
    K_h = np.zeros((wl.C,) + tuple(2 * n - 1 for n in wl.dims), dtype=np.float32)
    K_h[(slice(None),) + tuple(n - 1 + k for n, k in zip(wl.dims, s))] = 1.0
    _, rk = oracle.bwd_points(x_h, p.alpha, p.beta, K_h, dy_h, None, kp)
    del K_h
    dK_h = dK.cpu().numpy()
    errs["dK_pts"] = float(np.max(np.abs(np.array([dK_h[tuple(r)] for r in kp]) - rk)) / np.max(np.abs(rk)))
    print(f"[delta bwd] {name}: {errs}", flush=True)
    for k, v in errs.items():
        assert v <= (TOL[wl.dtype] if k.startswith("dx") else TOL_PARAM[wl.dtype]), (k, v)
