"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bar (element by element): max|y_gpu - y_ref| / max|y_ref| <= 1e-4 for fp32 I/O
and <= 2e-2 for bf16 I/O (fp32 FFT arithmetic in both cases).  Small grids are
compared in full against the direct sum; the five seeded workloads run at their
full sizes in the launch configuration the benchmark uses and are compared on
whole (b,c) slices against the FFT oracle and on sampled outputs against the
direct sum.
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


def _gpu_run(H, w, workspace=None):
    dev = torch.device("cuda:0")
    x = w["x"].to(dev)
    al = torch.from_numpy(w["alpha"]).to(dev)
    be = torch.from_numpy(w["beta"]).to(dev)
    kh = H.kernel_spectrum(w["K"].to(dev))
    y = H.fftconv_fwd(x, al, be, kh, workspace=workspace)
    torch.cuda.synchronize()
    return y, kh


SMALL = [
    ((2,), 1, 1, "f32"), ((64,), 3, 3, "f32"), ((1024,), 2, 3, "f32"), ((256,), 1, 5, "bf16"),
    ((2, 2), 1, 1, "f32"), ((4, 8), 2, 3, "f32"), ((8, 4), 1, 2, "f32"), ((32, 32), 1, 4, "f32"),
    ((16, 64), 2, 2, "f32"), ((64, 16), 1, 3, "bf16"), ((2, 512), 1, 2, "f32"), ((512, 2), 1, 2, "f32"),
    ((2, 2, 2), 1, 1, "f32"), ((4, 8, 16), 2, 3, "f32"), ((16, 4, 8), 1, 2, "f32"), ((8, 8, 8), 3, 1, "f32"),
    ((2, 2, 64), 1, 2, "f32"), ((64, 2, 2), 1, 2, "f32"), ((8, 16, 8), 2, 3, "bf16"),
    # 512-point out-axis lines (registers hold the first twiddled pass) with
    # fewer slots than a tile, and with two whole tiles
    ((256, 4), 2, 3, "f32"), ((256, 2), 1, 2, "bf16"), ((256, 32), 1, 2, "f32"),
    # 1024-point out-axis lines of a volume (4-line tiles, two mirrored rows)
    ((512, 2, 4), 1, 2, "f32"), ((512, 4, 16), 1, 1, "bf16"),
    # maximum extents: 2048-point transforms on every axis position
    ((1024, 2), 2, 2, "f32"), ((2, 1024), 1, 3, "bf16"), ((1024, 2, 2), 1, 2, "f32"), ((2, 1024, 2), 2, 1, "f32"),
    ((2, 2, 1024), 1, 2, "bf16"),
]


@pytest.mark.parametrize("dims,B,C,dtype", SMALL, ids=lambda v: str(v))
def test_small_grids_match_direct_sum(H, dims, B, C, dtype):
    w = synth.make(dims, B=B, C=C, dtype=dtype, seed=17 + sum(dims) + B + C)
    y, _ = _gpu_run(H, w)
    ref = oracle.direct(w["x"].float().numpy(), w["alpha"], w["beta"], w["K"].numpy())
    got = y.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert _rel(got, ref) <= TOL[dtype]


# (128, 8, 32) and (256, 4, 16): 256- and 512-point out-axis lines whose tiles
# take the row pairs fastest in the work-item order, with several row pairs
# and slot tiles per channel
@pytest.mark.parametrize("dims,B,C", [((128, 128), 2, 2), ((64, 256), 1, 2), ((32, 64, 16), 1, 2), ((512, 64), 1, 3),
                                      ((128, 8, 32), 2, 2), ((256, 4, 16), 1, 2)])
def test_medium_grids_match_fft_oracle(H, dims, B, C):
    w = synth.make(dims, B=B, C=C, dtype="f32", seed=5)
    y, _ = _gpu_run(H, w)
    ref = oracle.fftconv(w["x"].numpy(), w["alpha"], w["beta"], w["K"].numpy())
    assert _rel(y.cpu().numpy(), ref) <= 1e-4


@pytest.mark.parametrize("dims", [(16,), (64,), (8, 8), (4, 16), (32, 8), (4, 4, 4), (8, 4, 16), (2, 8, 4)])
def test_kernel_spectrum_layout(H, dims):
    """K_hat against the oracle's DFT of the wrap-placed kernel, in the library
    layout: main slots k_in >= 1 hold g*Khat, slot 0 holds g*(Khat0 + KhatS)/2,
    the trailing block g*(Khat0 - KhatS)/2, g = 1/(2 prod N); the main block is
    slot-tile-major, [S/T][N_out][N_mid][T]."""
    C = 3
    w = synth.make(dims, B=1, C=C, seed=3, dtype="f32")
    kh = H.kernel_spectrum(w["K"].to("cuda")).cpu().numpy().reshape(C, -1)
    d = len(dims)
    no, nm, ni = (1, 1, dims[0]) if d == 1 else ((dims[0], 1, dims[1]) if d == 2 else dims)
    No, Nm, Ni = (2 * no if d >= 2 else 1), (2 * nm if d == 3 else 1), 2 * ni
    S = ni
    full = oracle.kernel_spectrum(w["K"].numpy(), dims).reshape(C, No, Nm, Ni)
    g = 1.0 / (2 * No * Nm * Ni)
    T = H.spectrum_tile(dims)
    assert T >= 1 and S % T == 0 and (T & (T - 1)) == 0
    main = kh[:, :No * Nm * S].reshape(C, S // T, No, Nm, T).transpose(0, 2, 3, 1, 4).reshape(C, No, Nm, S)
    dblk = kh[:, No * Nm * S:].reshape(C, No, Nm)
    scale = np.abs(full).max() * g
    assert np.abs(main[..., 1:] - g * full[..., 1:S]).max() <= 1e-5 * scale
    assert np.abs(main[..., 0] - g * (full[..., 0] + full[..., S]) / 2).max() <= 1e-5 * scale
    assert np.abs(dblk - g * (full[..., 0] - full[..., S]) / 2).max() <= 1e-5 * scale


def test_chunked_workspace_is_bitwise_identical(H):
    dims, B, C = (64, 64), 3, 5
    w = synth.make(dims, B=B, C=C, seed=9)
    y_full, _ = _gpu_run(H, w)
    small = torch.empty(H.workspace_bytes(B, C, dims, minimum=True), dtype=torch.uint8, device="cuda")
    y_one, _ = _gpu_run(H, w, workspace=small)
    assert torch.equal(y_full, y_one)


def test_deterministic_and_workspace_poison_free(H):
    dims, B, C = (32, 16, 8), 2, 3
    w = synth.make(dims, B=B, C=C, seed=10)
    dev = "cuda"
    x, al, be = w["x"].to(dev), torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev)
    kh = H.kernel_spectrum(w["K"].to(dev))
    nb = H.workspace_bytes(B, C, dims)
    ws = torch.empty(nb // 4, dtype=torch.float32, device=dev)
    outs = []
    for fill in (0.0, float("nan"), float("inf"), 0.0):
        ws.fill_(fill)
        outs.append(H.fftconv_fwd(x, al, be, kh, workspace=ws.view(torch.uint8)).clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_runs_on_a_side_stream(H):
    dims, B, C = (32, 32), 2, 2
    w = synth.make(dims, B=B, C=C, seed=12)
    y0, _ = _gpu_run(H, w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1, _ = _gpu_run(H, w)
    s.synchronize()
    assert torch.equal(y0, y1)


def test_empty_batch(H):
    x = torch.empty((0, 3, 8, 8), device="cuda")
    al = torch.zeros(3, device="cuda")
    kh = H.kernel_spectrum(torch.zeros((3, 15, 15), device="cuda"))
    y = H.fftconv_fwd(x, al, al, kh)
    assert y.shape == x.shape


# ------------------------------------------------------------ full workloads

def _full_workload(H, wl, o2_pairs, sample_pairs, per_pair):
    dev = torch.device("cuda:0")
    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x_t = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype)
    K = synth.kernel_channels(wl.dims, p, device=dev)            # fp32 on the device
    kh = H.kernel_spectrum(K)
    x = x_t.to(dev)
    al, be = torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev)
    y = H.fftconv_fwd(x, al, be, kh)
    torch.cuda.synchronize()
    del kh
    K_h = K.cpu().numpy()
    del K
    x_h = x_t.float().numpy()
    y_h = y.float().cpu().numpy().reshape((wl.B * wl.C,) + wl.dims)
    ys = y_h.reshape((wl.B, wl.C) + wl.dims)
    errs = []
    scale = 0.0
    if o2_pairs:
        ref = oracle.fftconv(x_h, p.alpha, p.beta, K_h, pairs=o2_pairs)
        scale = float(np.max(np.abs(ref)))
        errs.append(float(np.max(np.abs(y_h[o2_pairs] - ref))))
    pts = synth.sample_points(wl.dims, wl.B, wl.C, sample_pairs, per_pair, seed=wl.seed)
    ref_pts = oracle.direct_points(x_h, p.alpha, p.beta, K_h, pts)
    got_pts = np.array([ys[tuple(r)] for r in pts])
    scale = max(scale, float(np.max(np.abs(ref_pts))))
    errs.append(float(np.max(np.abs(got_pts - ref_pts))))
    assert np.all(np.isfinite(y_h))
    return max(errs) / scale


def test_workload_2d_32(H):
    wl = synth.WORKLOADS[0]
    w = synth.make(wl)
    y, _ = _gpu_run(H, w)
    ref = oracle.direct(w["x"].numpy(), w["alpha"], w["beta"], w["K"].numpy())
    assert _rel(y.cpu().numpy(), ref) <= TOL[wl.dtype]


@pytest.mark.timeout(300)
def test_workload_2d_256(H):
    wl = synth.WORKLOADS[1]
    P = wl.B * wl.C
    err = _full_workload(H, wl, o2_pairs=[0, 77, P - 1], sample_pairs=[(0, 5), (7, 63), (3, 31)], per_pair=24)
    assert err <= TOL[wl.dtype]


@pytest.mark.timeout(300)
def test_workload_2d_1024_bf16(H):
    wl = synth.WORKLOADS[2]
    P = wl.B * wl.C
    err = _full_workload(H, wl, o2_pairs=[0, P - 1], sample_pairs=[(0, 64), (1, 127)], per_pair=8)
    assert err <= TOL[wl.dtype]


@pytest.mark.timeout(300)
def test_workload_3d_128(H):
    wl = synth.WORKLOADS[3]
    err = _full_workload(H, wl, o2_pairs=[0], sample_pairs=[(0, 13), (0, 31)], per_pair=16)
    assert err <= TOL[wl.dtype]


@pytest.mark.timeout(600)
def test_workload_3d_512_bf16(H):
    wl = synth.WORKLOADS[4]
    err = _full_workload(H, wl, o2_pairs=[], sample_pairs=[(0, 0), (0, 3)], per_pair=6)
    assert err <= TOL[wl.dtype]


@pytest.mark.timeout(600)
def test_workload_3d_512x512x64(H):
    wl = synth.WORKLOADS[7]
    err = _full_workload(H, wl, o2_pairs=[0], sample_pairs=[(0, 5), (0, 15)], per_pair=8)
    assert err <= TOL[wl.dtype]


@pytest.mark.timeout(600)
def test_workload_3d_1024x1024x256(H):
    wl = synth.WORKLOADS[8]
    err = _full_workload(H, wl, o2_pairs=[], sample_pairs=[(0, 0), (0, 1)], per_pair=4)
    assert err <= TOL[wl.dtype]


# ------------------------------------------------------- channel chunking

def test_launch_plan_and_balanced_chunks(H):
    minb = H.workspace_bytes(8, 64, (256, 256), torch.float32, minimum=True)
    assert H.launch_plan(8, 64, (256, 256), torch.float32, minb) == {"launches": 64 * 3, "chunk_channels": 1}
    assert H.launch_plan(8, 64, (256, 256), torch.float32, 16 * minb) == {"launches": 4 * 3, "chunk_channels": 16}
    # 64 channels with room for 30: three chunks of 22, 22, 20 rather than 30, 30, 4.
    assert H.launch_plan(8, 64, (256, 256), torch.float32, 30 * minb) == {"launches": 3 * 3, "chunk_channels": 22}
    assert H.launch_plan(1, 4, (8, 8, 8), torch.float32, 1 << 30)["launches"] == 5
    assert H.launch_plan(2, 3, (256,), torch.float32, 0)["launches"] == 1


@pytest.mark.parametrize("dims,B,C,dtype", [((32, 32), 2, 7, "f32"), ((64, 64, 64), 1, 5, "bf16")],
                         ids=lambda v: str(v))
def test_every_chunking_gives_the_same_output(H, dims, B, C, dtype):
    w = synth.make(dims, B=B, C=C, dtype=dtype, seed=40 + C)
    dt = w["x"].dtype
    minb = H.workspace_bytes(B, C, dims, dt, minimum=True)
    outs = []
    for k in (1, 2, 3, C):
        ws = torch.empty(k * minb, dtype=torch.uint8, device="cuda")
        outs.append(_gpu_run(H, w, workspace=ws)[0])
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_two_streams_do_not_share_a_workspace(H):
    """Same-shape calls in flight on two streams, each with the cached
    workspace of its own stream, give the results of eager single-stream calls."""
    dims, B, C = (128, 128), 2, 8
    dev = torch.device("cuda:0")
    runs = []
    for seed in (61, 62):
        w = synth.make(dims, B=B, C=C, seed=seed)
        x = w["x"].to(dev)
        al, be = torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev)
        kh = H.kernel_spectrum(w["K"].to(dev))
        runs.append((x, al, be, kh, H.fftconv_fwd(x, al, be, kh).clone()))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[], []]
    for _ in range(4):
        for k, s in enumerate(streams):
            with torch.cuda.stream(s):
                x, al, be, kh, _ = runs[k]
                outs[k].append(H.fftconv_fwd(x, al, be, kh))
    torch.cuda.synchronize()
    for k in range(2):
        for o in outs[k]:
            assert torch.equal(o, runs[k][4])


def test_released_workspaces_are_reallocated(H):
    """release_workspaces() empties the binding's workspace cache; the next
    call allocates a new buffer and gives the same result."""
    w = synth.make((128, 64), B=2, C=3, seed=41)
    dev = torch.device("cuda:0")
    x = w["x"].to(dev)
    al, be = torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev)
    kh = H.kernel_spectrum(w["K"].to(dev))
    y0 = H.fftconv_fwd(x, al, be, kh)
    assert H._ws_cache
    H.release_workspaces()
    assert not H._ws_cache
    y1 = H.fftconv_fwd(x, al, be, kh)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_bad_outputs_are_rejected_before_the_call(H):
    w = synth.make((16, 16), B=1, C=2, seed=3)
    dev = torch.device("cuda:0")
    x = w["x"].to(dev)
    al, be = torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev)
    kh = H.kernel_spectrum(w["K"].to(dev))
    with pytest.raises(TypeError):
        H.fftconv_fwd(x, al, be, kh, y=torch.empty(x.shape, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        H.fftconv_fwd(x, al, be, kh, y=torch.empty((1, 2, 16, 8), device=dev))
    with pytest.raises(ValueError):
        H.fftconv_fwd(x, al, be, kh, y=x)
    with pytest.raises(ValueError):
        H.kernel_spectrum(w["K"].to(dev), out=torch.empty(4, dtype=torch.complex64, device=dev))
    with pytest.raises(TypeError):   # a host workspace would reach the kernels as a device pointer
        H.fftconv_fwd(x, al, be, kh, workspace=torch.empty(H.workspace_bytes(1, 2, (16, 16)), dtype=torch.uint8))
    with pytest.raises(TypeError):
        H.fftconv_fwd(x, al.cpu(), be, kh)
    dy = torch.randn_like(x)
    with pytest.raises(ValueError):
        H.fftconv_bwd(x, al, be, kh, dy, dK=torch.empty((1, 2, 31, 31), device=dev))
    with pytest.raises(ValueError):
        H.fftconv_bwd(x, al, be, kh, dy, dx=dy)
