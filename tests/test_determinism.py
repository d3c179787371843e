"""Run-to-run determinism: every path repeated 20 times on the same inputs,
with the workspace refilled before each call by a different poison pattern
(zeros, NaN, +/-inf, huge values, random bits), must give bit-identical
outputs.  The kernels sum in fixed orders (no atomics, no order that depends
on scheduling) and write every workspace value before reading it."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

REPEATS = 20


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dimensional_fft_long_amd as H

    H.get_lib()
    return H


def _poison(ws: torch.Tensor, k: int):
    f = ws.view(torch.float32)
    kind = k % 5
    if kind == 0:
        f.zero_()
    elif kind == 1:
        f.fill_(float("nan"))
    elif kind == 2:
        f.fill_(float("inf") if k % 2 else -float("inf"))
    elif kind == 3:
        f.fill_(3.0e38)
    else:
        g = torch.Generator(device=ws.device).manual_seed(k)
        ws.view(torch.int32).random_(-2**31, 2**31 - 1, generator=g)


def _inputs(dims, B, C, dtype, seed):
    w = synth.make(dims, B=B, C=C, dtype=dtype, seed=seed)
    dev = "cuda"
    return (w["x"].to(dev), torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev),
            w["K"].to(dev))


def _repeat(call, ws):
    outs = []
    for k in range(REPEATS):
        if ws is not None:
            _poison(ws, k)
        outs.append([t.clone() for t in call()])
    torch.cuda.synchronize()
    for k, o in enumerate(outs[1:], 1):
        for i, (g, r) in enumerate(zip(o, outs[0])):
            assert torch.equal(g, r), f"repeat {k}, output {i} differs"


FWD = [((128, 64), 2, 3, "f32"),      # three passes, 256-point out-axis lines
       ((32, 32), 2, 3, "f32"),       # on-chip 2-D
       ((16, 8, 32), 2, 3, "bf16"),   # five passes
       ((1 << 16,), 1, 2, "f32"),     # long 1-D
       ((512,), 3, 4, "bf16")]        # one-launch 1-D


@pytest.mark.parametrize("dims,B,C,dtype", FWD)
def test_forward_repeats_bitwise(H, dims, B, C, dtype):
    x, al, be, K = _inputs(dims, B, C, dtype, seed=31)
    kh = H.kernel_spectrum(K)
    nb = H.workspace_bytes(B, C, dims, x.dtype)
    ws = torch.empty(max(nb, 8), dtype=torch.uint8, device="cuda") if nb else None
    y = torch.empty_like(x)
    _repeat(lambda: [H.fftconv_fwd(x, al, be, kh, y=y, workspace=ws)], ws)


def test_circular_forward_repeats_bitwise(H):
    dims, B, C = (64, 32), 2, 3
    w = synth.make(dims, B=B, C=C, seed=32, with_kernel=False)
    dev = "cuda"
    x, al, be = w["x"].to(dev), torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev)
    kh = H.kernel_spectrum_circ(synth.circular_kernel(dims, w["params"], device=dev))
    ws = torch.empty(H.circ_workspace_bytes(B, C, dims), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    _repeat(lambda: [H.fftconv_fwd_circ(x, al, be, kh, y=y, workspace=ws)], ws)


BWD = [((64, 32), 3, 2, "f32"), ((8, 8, 16), 2, 2, "f32"), ((1 << 14,), 2, 2, "bf16"), ((256,), 4, 3, "f32")]


@pytest.mark.parametrize("dims,B,C,dtype", BWD)
def test_backward_repeats_bitwise(H, dims, B, C, dtype):
    x, al, be, K = _inputs(dims, B, C, dtype, seed=33)
    dy = synth.draw_dy(dims, B, C, dtype, 34).to("cuda")
    kh = H.kernel_spectrum(K)
    ws = torch.empty(H.bwd_workspace_bytes(B, C, dims, x.dtype), dtype=torch.uint8, device="cuda")
    _repeat(lambda: H.fftconv_bwd(x, al, be, kh, dy, workspace=ws), ws)


def test_generator_repeats_bitwise(H):
    dims, B, C = (32, 64), 2, 3
    x, al, be, _ = _inputs(dims, B, C, "f32", seed=35)
    gen = {k: (torch.from_numpy(v).cuda() if isinstance(v, np.ndarray) else v)
           for k, v in synth.draw_generator(dims, C, 36).items()}
    ws = torch.empty(H.generate_workspace_bytes(B, C, dims), dtype=torch.uint8, device="cuda")
    kh = torch.empty(H.spectrum_bytes(B * C, dims) // 8, dtype=torch.complex64, device="cuda").view(B * C, -1)
    y = torch.empty_like(x)
    fw = torch.empty(max(H.workspace_bytes(B, C, dims), 8), dtype=torch.uint8, device="cuda")

    def call():
        H.generate_kernel_spectrum(x, gen, out=kh, workspace=ws)
        return [kh, H.fftconv_fwd_per_sample(x, al, be, kh, y=y, workspace=fw)]

    _repeat(call, ws)
