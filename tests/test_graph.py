"""HIP graph capture of the entry points.

Every entry point only enqueues kernels on the caller's stream (no
allocation, copy, memset or synchronisation inside), so a whole forward and
backward can be captured once into a graph and replayed.  Each test captures
with caller-owned workspaces, replays the graph several times with new inputs
written in eagerly between the replays (and eager work of other kernels in
between), and checks every replay against an eager call on the same inputs:
the same kernels in the same order give the same bits.
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dimensional_fft_long_amd as H

    H.get_lib()
    return H


@pytest.mark.parametrize("dims,B,C", [((64, 64), 2, 3), ((16, 32, 8), 2, 2), ((4096,), 2, 2)],
                         ids=lambda v: str(v))
def test_forward_and_backward_replay_like_eager_calls(H, dims, B, C):
    dev = torch.device("cuda:0")
    p = synth.draw_params(dims, C, 77)
    x = synth.draw_x(p.rng, B, C, dims, "f32").to(dev)
    dy = synth.draw_dy(dims, B, C, "f32", 77).to(dev)
    K = synth.kernel_channels(dims, p, device=dev)
    al, be = torch.from_numpy(p.alpha).to(dev), torch.from_numpy(p.beta).to(dev)
    kh = H.kernel_spectrum(K)
    ws_f = torch.empty(max(H.workspace_bytes(B, C, dims), 8), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(H.bwd_workspace_bytes(B, C, dims), 8), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    outs = (torch.empty_like(x), torch.empty(C, device=dev), torch.empty(C, device=dev),
            torch.empty((C,) + tuple(2 * n - 1 for n in dims), device=dev))

    def step():
        H.fftconv_fwd(x, al, be, kh, y=y, workspace=ws_f)
        H.fftconv_bwd(x, al, be, kh, dy, *outs, workspace=ws_b)

    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(5)
    for rep in range(3):
        x.copy_(torch.randn(x.shape, generator=gen).to(dev))
        dy.copy_(torch.randn(dy.shape, generator=gen).to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [y.clone()] + [t.clone() for t in outs]
        _ = (x * 2.0).sum()  # unrelated eager work between replays
        step()
        torch.cuda.synchronize()
        want = [y] + list(outs)
        for a, b in zip(got, want):
            assert torch.equal(a, b), rep
