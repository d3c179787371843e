"""The allocation-free forward (hyenand_fftconv_fwd_noalloc) against the
workspace forward (hyenand_fftconv_fwd), both through the C ABI: two calls in
a row, the second with a smaller input, each compared with the workspace
forward on the same inputs (the same kernels run in other channel chunks, so
the results agree bit for bit; the bar of the parity tests, max|d|/max|y| <=
1e-4 for fp32 and 2e-2 for bf16 I/O, is implied)."""
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


def _inputs(H, dims, B, C, dtype, seed):
    dev = torch.device("cuda:0")
    w = synth.make(dims, B=B, C=C, dtype=dtype, seed=seed)
    x = w["x"].to(dev)
    al, be = torch.from_numpy(w["alpha"]).to(dev), torch.from_numpy(w["beta"]).to(dev)
    kh = H.kernel_spectrum(w["K"].to(dev))
    return x, al, be, kh


@pytest.mark.parametrize("big,small", [
    (((256, 256), 8, 20, "f32"), ((32, 256), 2, 3, "f32")),          # 20 channels: two 64 MiB chunks
    (((64, 64, 64), 2, 5, "bf16"), ((16, 8, 32), 1, 2, "bf16")),
], ids=["2d", "3d"])
def test_noalloc_matches_workspace_forward_twice(H, big, small):
    torch.cuda.synchronize()
    for dims, B, C, dtype in (big, small):
        print(f"[noalloc] dims={dims} B={B} C={C} {dtype}", flush=True)
        x, al, be, kh = _inputs(H, dims, B, C, dtype, seed=sum(dims) + C)
        ref = H.fftconv_fwd(x, al, be, kh)
        y = torch.full_like(x, float("nan"))
        H.fftconv_fwd_noalloc(x, al, be, kh, y)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


def test_noalloc_rejects_a_channel_beyond_the_scratch(H):
    dims, B, C = (512, 512, 512), 1, 1          # one channel needs 2 GiB of workspace
    assert H.workspace_bytes(B, C, dims, torch.bfloat16, minimum=True) > H.noalloc_max_workspace()
    dev = torch.device("cuda:0")
    x = torch.zeros((B, C) + dims, dtype=torch.bfloat16, device=dev)
    al = torch.zeros(C, device=dev)
    kh = torch.zeros(H.spectrum_bytes(C, dims) // 8, dtype=torch.complex64, device=dev)
    with pytest.raises(H.HyenandError) as e:
        H.fftconv_fwd_noalloc(x, al, al, kh, torch.empty_like(x))
    assert e.value.code == H.ERR_WORKSPACE
