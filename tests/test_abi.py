"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments before anything is launched (no GPU needed: every call
here returns from argument validation or a size query)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hyenand.h")


@pytest.fixture(scope="module")
def H():
    import dimensional_fft_long_amd as H

    if not os.path.exists(H.LIB_PATH):
        from dimensional_fft_long_amd import build

        build.build()
    H.get_lib()
    return H


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(hyenand_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(H):
    names = _declared()
    assert "hyenand_fftconv_fwd" in names and "hyenand_kernel_spectrum" in names
    lib = H.get_lib()
    for nm in names:
        assert hasattr(lib, nm), nm
    assert set(names) == set(H.EXPORTS)


def _dims(*v):
    return (ctypes.c_int64 * len(v))(*v)


def test_status_strings_and_version(H):
    lib = H.get_lib()
    assert lib.hyenand_version() >= 100
    seen = {lib.hyenand_status_string(c) for c in range(5)}
    assert len(seen) == 5
    assert lib.hyenand_status_string(99) == b"unknown status"


def test_sizes(H):
    lib = H.get_lib()
    # 2-D 256x256, C=64: main N0*S = 512*256, dblk N0 = 512, complex64.
    assert lib.hyenand_kernel_spectrum_bytes(64, 2, _dims(256, 256)) == 64 * (512 * 256 + 512) * 8
    # 3-D 128^3: main 256*256*128, dblk 256*256.
    assert lib.hyenand_kernel_spectrum_bytes(32, 3, _dims(128, 128, 128)) == 32 * (256 * 256 * 128 + 256 * 256) * 8
    # 1-D 64: main 64, dblk 1.
    assert lib.hyenand_kernel_spectrum_bytes(3, 1, _dims(64)) == 3 * 65 * 8
    # Workspace per pair n0 * N_mid * S complex; minimum is one channel (all B).
    assert lib.hyenand_fftconv_workspace_min_bytes(8, 64, 2, _dims(256, 256), 0) == 8 * 256 * 256 * 8
    assert lib.hyenand_fftconv_workspace_min_bytes(1, 4, 3, _dims(512, 512, 512), 1) == 512 * 1024 * 512 * 8
    rec = lib.hyenand_fftconv_workspace_bytes(8, 64, 2, _dims(256, 256), 0)
    assert rec % (8 * 256 * 256 * 8) == 0 and 0 < rec <= 64 * 8 * 256 * 256 * 8
    assert rec == lib.hyenand_fftconv_workspace_bytes(8, 64, 2, _dims(256, 256), 0)
    assert lib.hyenand_fftconv_workspace_bytes(4, 4, 1, _dims(1024), 0) == 0  # 1-D needs none
    # Unsupported shapes size to 0.
    for d, dims in [(2, _dims(3, 4)), (2, _dims(1, 4)), (1, _dims(1 << 25)), (1, _dims(3 << 11)), (4, _dims(2, 2, 2, 2))]:
        assert lib.hyenand_kernel_spectrum_bytes(2, d, dims) == 0
        assert lib.hyenand_kernel_spectrum_tile(d, dims) == 0


def test_spectrum_slot_tile(H):
    """The K_hat slot tile: the out-axis workgroup's tile width capped at S, a
    power of two dividing S (1-D: the whole row)."""
    lib = H.get_lib()
    assert lib.hyenand_kernel_spectrum_tile(2, _dims(256, 256)) == 8       # 512-point out lines: 8-line tiles
    assert lib.hyenand_kernel_spectrum_tile(2, _dims(1024, 1024)) == 8     # 2048-point: 16384 / 2048
    assert lib.hyenand_kernel_spectrum_tile(2, _dims(512, 4)) == 4         # capped at S = 4
    assert lib.hyenand_kernel_spectrum_tile(3, _dims(128, 128, 128)) == 16  # 256-point, two mirrored rows
    assert lib.hyenand_kernel_spectrum_tile(3, _dims(512, 512, 512)) == 64   # 8-line out tiles: 64-slot tiles
    assert lib.hyenand_kernel_spectrum_tile(1, _dims(64)) == 64
    for d in (1, 2, 3):
        for e in range(1, 11):
            dims = _dims(*([2 ** e] * d))
            t = lib.hyenand_kernel_spectrum_tile(d, dims)
            S = 2 ** e
            assert t >= 1 and S % t == 0 and t & (t - 1) == 0


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation first
MISALIGNED = ctypes.c_void_p(0x10001)


@pytest.mark.parametrize("d,dims,code", [
    (0, (4,), 2), (4, (4, 4, 4, 4), 2), (2, (3, 4), 2), (2, (4, 1), 2), (2, (2048, 2), 2), (1, (6,), 2),
])
def test_fwd_rejects_shapes(H, d, dims, code):
    lib = H.get_lib()
    rc = lib.hyenand_fftconv_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, d, _dims(*dims), 0, FAKE, 1 << 30, None)
    assert rc == code


def test_fwd_rejects_arguments(H):
    lib = H.get_lib()
    dd = _dims(8, 8)
    ws = 1 << 20
    call = lambda x=FAKE, a=FAKE, b=FAKE, k=FAKE, y=FAKE, B=1, C=1, dt=0, w=FAKE, wb=ws: \
        lib.hyenand_fftconv_fwd(x, a, b, k, y, B, C, 2, dd, dt, w, wb, None)
    assert call(x=None) == 1
    assert call(y=None) == 1
    assert call(k=None) == 1
    assert call(a=None) == 1
    assert call(B=-1) == 1
    assert call(C=-2) == 1
    assert call(dt=7) == 1
    assert call(x=MISALIGNED) == 1
    assert call(k=MISALIGNED) == 1
    # A grid that needs a workspace (an axis above 128: the multi-pass kernels).
    dw = _dims(8, 256)
    callw = lambda w=FAKE, wb=ws: lib.hyenand_fftconv_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 2, dw, 0, w, wb, None)
    assert callw(w=None) == 3
    assert callw(wb=8 * 256 * 8 - 1) == 3        # one pair needs n0 * S * 8 = 16384 bytes
    assert callw(w=MISALIGNED) == 1
    # Empty calls succeed without touching anything.
    assert call(x=None, y=None, B=0) == 0
    assert call(x=None, y=None, C=0) == 0
    # dims = NULL
    assert lib.hyenand_fftconv_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 2, None, 0, FAKE, ws, None) == 1


def test_spectrum_rejects_arguments(H):
    lib = H.get_lib()
    assert lib.hyenand_kernel_spectrum(FAKE, FAKE, -1, 2, _dims(8, 8), None) == 1
    assert lib.hyenand_kernel_spectrum(None, FAKE, 2, 2, _dims(8, 8), None) == 1
    assert lib.hyenand_kernel_spectrum(FAKE, None, 2, 2, _dims(8, 8), None) == 1
    assert lib.hyenand_kernel_spectrum(FAKE, MISALIGNED, 2, 2, _dims(8, 8), None) == 1
    assert lib.hyenand_kernel_spectrum(FAKE, FAKE, 2, 2, _dims(8, 12), None) == 2
    assert lib.hyenand_kernel_spectrum(FAKE, FAKE, 2, 5, _dims(8, 8), None) == 2
    assert lib.hyenand_kernel_spectrum(None, None, 0, 2, _dims(8, 8), None) == 0


def test_bwd_sizes(H):
    lib = H.get_lib()
    # 2-D 256x256, B=8: per channel two planes of B * n0 * S complex, the
    # kernel-gradient spectrum N0 * S complex and one float2 per line pair.
    plane = 8 * 256 * 256 * 8
    per_ch = 2 * plane + 512 * 256 * 8 + 8 * 128 * 8
    assert lib.hyenand_fftconv_bwd_workspace_min_bytes(8, 64, 2, _dims(256, 256), 0, 1) == per_ch
    assert lib.hyenand_fftconv_bwd_workspace_min_bytes(8, 64, 2, _dims(256, 256), 0, 0) == plane + 8 * 128 * 8
    rec = lib.hyenand_fftconv_bwd_workspace_bytes(8, 64, 2, _dims(256, 256), 0, 1)
    assert rec % per_ch == 0 and per_ch <= rec <= 64 * per_ch
    # 1-D: per pair S complex for the kernel gradient and one float2.
    assert lib.hyenand_fftconv_bwd_workspace_min_bytes(4, 2, 1, _dims(64), 0, 1) == 4 * 64 * 8 + 4 * 8
    assert lib.hyenand_fftconv_bwd_workspace_min_bytes(4, 2, 1, _dims(64), 0, 0) == 4 * 8
    for d, dims in [(2, _dims(3, 4)), (1, _dims(1 << 25))]:
        assert lib.hyenand_fftconv_bwd_workspace_bytes(2, 2, d, dims, 0, 1) == 0


def test_bwd_rejects_arguments(H):
    lib = H.get_lib()
    dd = _dims(8, 8)
    ws = 1 << 20
    call = lambda x=FAKE, a=FAKE, b=FAKE, k=FAKE, dy=FAKE, dx=FAKE, da=FAKE, db=FAKE, dK=FAKE, B=1, C=1, d=2, \
        dims=dd, dt=0, w=FAKE, wb=ws: lib.hyenand_fftconv_bwd(x, a, b, k, dy, dx, da, db, dK, B, C, d, dims, dt,
                                                              w, wb, None)
    for kw in ("x", "a", "b", "k", "dy", "dx", "da", "db"):
        assert call(**{kw: None}) == 1, kw
    assert call(B=-1) == 1 and call(C=-1) == 1 and call(dt=3) == 1
    assert call(x=MISALIGNED) == 1 and call(dy=MISALIGNED) == 1 and call(dx=MISALIGNED) == 1
    assert call(k=MISALIGNED) == 1 and call(dK=MISALIGNED) == 1 and call(w=MISALIGNED) == 1
    assert call(w=None) == 3
    need = lib.hyenand_fftconv_bwd_workspace_min_bytes(1, 1, 2, dd, 0, 1)
    assert call(wb=need - 1) == 3
    assert call(d=2, dims=_dims(8, 6)) == 2 and call(d=0) == 2 and call(dims=None) == 1
    assert call(x=None, dy=None, dx=None, C=0) == 0


def test_circular_sizes_and_rejects(H):
    lib = H.get_lib()
    # 2-D 256x256 circular: N = n, S = 128; main N0 * S = 256 * 128, dblk N0 = 256.
    assert lib.hyenand_kernel_spectrum_circ_bytes(4, 2, _dims(256, 256)) == 4 * (256 * 128 + 256) * 8
    assert lib.hyenand_kernel_spectrum_circ_bytes(2, 3, _dims(8, 8, 8)) == 2 * (8 * 8 * 4 + 8 * 8) * 8
    assert lib.hyenand_kernel_spectrum_circ_bytes(3, 1, _dims(64)) == 3 * (32 + 1) * 8
    # workspace per pair n0 * N_mid * S with N_mid = n_mid
    assert lib.hyenand_fftconv_circ_workspace_min_bytes(2, 3, 2, _dims(64, 32), 0) == 2 * 64 * 16 * 8
    assert lib.hyenand_fftconv_circ_workspace_min_bytes(1, 1, 3, _dims(8, 16, 32), 0) == 8 * 16 * 16 * 8
    # n = 2 has no circular transform here (length >= 4); non-powers of two are unsupported
    for d, dims in [(1, _dims(2)), (2, _dims(4, 2)), (2, _dims(12, 8)), (1, _dims(2048))]:
        assert lib.hyenand_kernel_spectrum_circ_bytes(1, d, dims) == 0
        assert lib.hyenand_kernel_spectrum_circ_tile(d, dims) == 0
    for d in (1, 2, 3):
        for e in range(2, 11):
            t = lib.hyenand_kernel_spectrum_circ_tile(d, _dims(*([2 ** e] * d)))
            S = 2 ** (e - 1)
            assert t >= 1 and S % t == 0
    dd = _dims(8, 8)
    call = lambda x=FAKE, k=FAKE, y=FAKE, B=1, C=1, d=2, dims=dd, dt=0, w=FAKE, wb=1 << 20: \
        lib.hyenand_fftconv_fwd_circ(x, FAKE, FAKE, k, y, B, C, d, dims, dt, w, wb, None)
    assert call(x=None) == 1 and call(y=None) == 1 and call(k=MISALIGNED) == 1 and call(dt=5) == 1
    assert call(dims=_dims(2, 8)) == 2 and call(w=None) == 3 and call(wb=8 * 4 * 8 - 1) == 3
    assert call(x=None, y=None, B=0) == 0
    assert lib.hyenand_kernel_spectrum_circ(FAKE, FAKE, 2, 2, _dims(8, 2), None) == 2
    assert lib.hyenand_kernel_spectrum_circ(None, FAKE, 2, 2, _dims(8, 8), None) == 1


def test_circular_bwd_sizes_and_rejects(H):
    lib = H.get_lib()
    # 2-D 64x32 circular, B=2: per channel two planes of B * n0 * S complex
    # (S = 16), the kernel-gradient spectrum N0 * S and B * n0 / 2 float2.
    assert lib.hyenand_fftconv_bwd_circ_workspace_min_bytes(2, 3, 2, _dims(64, 32), 0, 1) == \
        (2 * 2 * 64 * 16 + 64 * 16 + 2 * 32) * 8
    assert lib.hyenand_fftconv_bwd_circ_workspace_min_bytes(2, 3, 2, _dims(64, 32), 0, 0) == (2 * 64 * 16 + 2 * 32) * 8
    # 1-D 64 circular, B=4: B * S complex (S = 32) and one float2 per signal
    assert lib.hyenand_fftconv_bwd_circ_workspace_min_bytes(4, 2, 1, _dims(64), 0, 1) == (4 * 32 + 4) * 8
    rec = lib.hyenand_fftconv_bwd_circ_workspace_bytes(2, 3, 2, _dims(64, 32), 1, 1)
    assert rec == 3 * (2 * 2 * 64 * 16 + 64 * 16 + 2 * 32) * 8
    for d, dims in [(1, _dims(2)), (2, _dims(4, 2)), (2, _dims(12, 8)), (1, _dims(2048))]:
        assert lib.hyenand_fftconv_bwd_circ_workspace_bytes(1, 1, d, dims, 0, 1) == 0
    dd = _dims(8, 8)
    call = lambda x=FAKE, dy=FAKE, dx=FAKE, da=FAKE, B=1, C=1, d=2, dims=dd, dt=0, w=FAKE, wb=1 << 20: \
        lib.hyenand_fftconv_bwd_circ(x, FAKE, FAKE, FAKE, dy, dx, da, FAKE, FAKE, B, C, d, dims, dt, w, wb, None)
    assert call(x=None) == 1 and call(dy=None) == 1 and call(dx=MISALIGNED) == 1 and call(da=None) == 1
    assert call(dims=_dims(2, 8)) == 2 and call(d=1, dims=_dims(4096)) == 2 and call(w=None) == 3
    need = lib.hyenand_fftconv_bwd_circ_workspace_min_bytes(1, 1, 2, dd, 0, 1)
    assert need > 0 and call(wb=need - 1) == 3
    assert call(x=None, dy=None, dx=None, C=0) == 0


def test_per_sample_bwd_rejects(H):
    lib = H.get_lib()
    dd = _dims(8, 8)
    call = lambda x=FAKE, dy=FAKE, dx=FAKE, db=FAKE, B=2, C=1, d=2, dims=dd, dt=0, w=FAKE, wb=1 << 20: \
        lib.hyenand_fftconv_bwd_per_sample(x, FAKE, FAKE, FAKE, dy, dx, FAKE, db, FAKE, B, C, d, dims, dt, w, wb, None)
    assert call(x=None) == 1 and call(dy=None) == 1 and call(dx=MISALIGNED) == 1 and call(db=None) == 1
    assert call(dims=_dims(8, 6)) == 2 and call(d=1, dims=_dims(1 << 25)) == 2 and call(w=None) == 3
    # the workspace of a batch of one is enough, whatever B
    need = lib.hyenand_fftconv_bwd_workspace_min_bytes(1, 1, 2, dd, 0, 1)
    assert call(wb=need - 1) == 3
    assert call(x=None, dy=None, dx=None, C=0) == 0


def test_long_1d_sizes(H):
    """1-D signals longer than 1024 take the long path: the full N = 2n complex
    spectrum per channel (no Nyquist packing), N complex of workspace per pair,
    three launches per channel chunk; the backward's workspace holds two
    planes per pair, the kernel-gradient plane and one partial sum per
    inverse-column workgroup; no circular mode."""
    lib = H.get_lib()
    # n -> partial sums per pair: N2 / TW with N2 the row length and TW the column tile
    for n, parts in ((2048, 1024 // 16), (1 << 16, 2048 // 16), (1 << 21, 2048 // 8), (1 << 23, 4096 // 4),
                     (1 << 24, 8192 // 4)):
        N = 2 * n
        assert lib.hyenand_kernel_spectrum_bytes(3, 1, _dims(n)) == 3 * N * 8
        assert lib.hyenand_fftconv_workspace_min_bytes(2, 3, 1, _dims(n), 0) == 2 * N * 8
        assert lib.hyenand_fftconv_bwd_workspace_min_bytes(2, 3, 1, _dims(n), 0, 1) == (2 * 2 * N + N + 2 * parts) * 8
        assert lib.hyenand_fftconv_bwd_workspace_min_bytes(2, 3, 1, _dims(n), 0, 0) == (2 * N + 2 * parts) * 8
        assert lib.hyenand_kernel_spectrum_circ_bytes(3, 1, _dims(n)) == 0
    import torch

    assert H.launch_plan(1, 4, (1 << 20,), torch.float32, 1 << 30)["launches"] == 3
    assert H.launch_plan(2, 4, (1 << 20,), torch.float32, 2 * 2 * (1 << 20) * 8)["launches"] == 4 * 3
    bw = lib.hyenand_fftconv_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, _dims(4096), 0, FAKE,
                                 1024, None)
    assert bw == 3  # accepted shape, workspace below one channel
    assert lib.hyenand_fftconv_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, _dims(1 << 25), 0,
                                   FAKE, 1 << 30, None) == 2


def test_output_checks_reject_bad_outputs(H):
    """Caller-provided outputs and workspaces are checked before any call:
    dtype, device, contiguity, exact shape, and no overlap with the input they
    must not alias (host tensors here; the GPU entry points run the same
    checks)."""
    import torch

    x = torch.zeros(2, 3, 8, 8)
    ok = torch.zeros(2, 3, 8, 8)
    assert H._check_out(ok, "y", x.shape, x.dtype, x.device, like=x) is ok
    with pytest.raises(TypeError):
        H._check_out(torch.zeros(2, 3, 8, 8, dtype=torch.bfloat16), "y", x.shape, x.dtype, x.device)
    with pytest.raises(ValueError):
        H._check_out(torch.zeros(2, 3, 8, 4), "y", x.shape, x.dtype, x.device)  # undersized
    with pytest.raises(ValueError):
        H._check_out(torch.zeros(2, 3, 8, 16), "y", x.shape, x.dtype, x.device)
    with pytest.raises(TypeError):
        H._check_out(torch.zeros(2, 3, 8, 16)[..., ::2], "y", x.shape, x.dtype, x.device)  # not contiguous
    with pytest.raises(ValueError):
        H._check_out(x, "y", x.shape, x.dtype, x.device, like=x)                      # aliases x
    with pytest.raises(ValueError):
        H._check_out(x.view(-1)[5:5 + 16], "dalpha", (16,), x.dtype, x.device, like=x)  # overlaps x
    with pytest.raises(TypeError):
        H._check_out(torch.zeros(3, dtype=torch.float64), "dalpha", (3,), torch.float32, x.device)
    with pytest.raises(ValueError):   # a per-sample-shaped dK where the shared one is expected
        H._check_out(torch.zeros(2, 3, 15, 15), "dK", (3, 15, 15), torch.float32, x.device)
    assert H._ws_bytes(torch.zeros(16, dtype=torch.uint8), x.device) == 16
    H.release_workspaces()   # an empty cache: nothing to synchronise
    assert H._ws_bytes(torch.zeros(4, dtype=torch.float64), x.device) == 32
    with pytest.raises(TypeError):   # a workspace on another device
        H._ws_bytes(torch.zeros(16, dtype=torch.uint8, device="meta"), x.device)
    with pytest.raises(TypeError):
        H._ws_bytes(torch.zeros(32, dtype=torch.uint8)[::2], x.device)
    with pytest.raises(TypeError):
        H._ws_bytes(bytearray(16), x.device)
    H._check_spectrum_out(torch.zeros(10, dtype=torch.complex64), 80, x.device)
    with pytest.raises(ValueError):
        H._check_spectrum_out(torch.zeros(9, dtype=torch.complex64), 80, x.device)
    with pytest.raises(TypeError):
        H._check_spectrum_out(torch.zeros(20, dtype=torch.float32), 80, x.device)


def test_library_does_not_load_the_oracle():
    """The product package never imports the oracle (it must fail loudly, not
    fall back, when its HIP library is missing)."""
    import subprocess
    import sys

    code = ("import sys; sys.path.insert(0, %r); import dimensional_fft_long_amd as H; "
            "print('oracle' in sys.modules)") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True).stdout
    assert out.strip() == "False"


EXTENTS_FUSED = (4, 8, 16, 32, 64)


def test_fused_shapes_take_one_launch_and_no_workspace(H):
    """Zero-padded 2-D grids with both extents in [4, 64] run the on-chip
    forward: one launch for every pair and no workspace."""
    import torch

    for n0 in EXTENTS_FUSED:
        for n1 in EXTENTS_FUSED:
            assert H.uses_fused2d((n0, n1))
            assert H.workspace_bytes(8, 64, (n0, n1), minimum=True) == 0
            assert H.workspace_bytes(8, 64, (n0, n1)) == 0
            assert H.launch_plan(8, 64, (n0, n1), torch.float32, 0) == {"launches": 1, "chunk_channels": 64}
    for dims in [(2, 8), (8, 2), (128, 128), (128, 64), (64, 128), (256, 256)]:
        assert not H.uses_fused2d(dims)
        assert H.workspace_bytes(2, 3, dims, minimum=True) > 0
    # the backward and the circular mode keep their multi-pass kernels
    assert H.bwd_workspace_bytes(2, 3, (32, 32), minimum=True) > 0
    assert H.circ_workspace_bytes(2, 3, (32, 32), minimum=True) > 0


def _gen_struct(H, R=4, D=8, p=FAKE):
    return H._Generator(R, D, *([p.value] * 10), 10.0)


def test_generator_sizes_and_rejects(H):
    """The generator's entry points: workspace sizes, and every argument check
    returns before a launch (FAKE pointers are never dereferenced)."""
    lib = H.get_lib()
    d2 = _dims(32, 64)
    ws = H.generate_workspace_bytes(2, 3, (32, 64))
    assert ws > 0 and ws % 256 == 0
    assert lib.hyenand_generate_workspace_bytes(2, 0, 2, d2) == 0
    assert lib.hyenand_generate_workspace_bytes(1, 1, 1, _dims(4096)) == 0  # long 1-D: not generated
    g = _gen_struct(H)
    call = lambda gen=ctypes.byref(g), x=FAKE, k=FAKE, B=2, C=3, d=2, dd=d2, dt=0, w=FAKE, wb=ws: \
        lib.hyenand_generate_kernel_spectrum(x, gen, k, B, C, d, dd, dt, w, wb, None)
    assert call(gen=None) == 1
    assert call(x=None) == 1
    assert call(k=None) == 1
    assert call(x=MISALIGNED) == 1
    assert call(dt=5) == 1
    assert call(B=-1) == 1
    assert call(C=8193) == 1                          # the sample's means live in LDS
    assert call(d=4) == 2
    assert call(d=1, dd=_dims(4096)) == 2            # the long 1-D path has no generator
    assert call(dd=_dims(32, 48)) == 2               # not a power of two
    assert call(w=None) == 3
    assert call(wb=ws - 1) == 3
    assert call(w=ctypes.c_void_p(0x10000 + 64)) == 1  # the workspace must be 256-byte aligned
    assert call(x=None, k=None, B=0) == 0
    for R, D in ((0, 8), (65, 8), (4, 0), (4, 65)):
        bad = _gen_struct(H, R, D)
        assert call(gen=ctypes.byref(bad)) == 1
    nulls = _gen_struct(H, p=ctypes.c_void_p(0))
    assert call(gen=ctypes.byref(nulls)) == 1
    mis = _gen_struct(H, p=MISALIGNED)
    assert call(gen=ctypes.byref(mis)) == 1


def test_generated_forward_sizes_and_rejects(H):
    lib = H.get_lib()
    dims = (32, 256)                                   # a multi-pass shape: the forward needs its workspace
    dd = _dims(*dims)
    gw = H.generate_workspace_bytes(2, 3, dims)
    rec = H.generated_workspace_bytes(2, 3, dims)
    mn = H.generated_workspace_bytes(2, 3, dims, minimum=True)
    fmin = H.workspace_bytes(2, 3, dims, minimum=True)
    assert mn == gw + fmin and rec >= mn
    # The on-chip 2-D forward needs no workspace of its own.
    assert H.generated_workspace_bytes(2, 3, (32, 32)) == H.generate_workspace_bytes(2, 3, (32, 32))
    g = _gen_struct(H)
    call = lambda gen=ctypes.byref(g), a=FAKE, y=FAKE, B=2, C=3, w=FAKE, wb=rec: \
        lib.hyenand_fftconv_fwd_generated(FAKE, a, FAKE, gen, FAKE, y, B, C, 2, dd, 0, w, wb, None)
    assert call(gen=None) == 1
    assert call(a=None) == 1
    assert call(y=None) == 1
    assert call(y=MISALIGNED) == 1
    assert call(w=None) == 3
    assert call(wb=gw - 8) == 3                       # not even the generator's region
    assert call(wb=mn - 8) == 3                       # the generator's region but not one forward chunk
    assert call(B=0, y=None) == 0


def test_generator_rejects_grids_beyond_the_launch_limit(H):
    """B C x (blocks of 128 spectrum rows) at 2^31 workgroups or more is refused
    before anything is launched (3-D 1024^3: 32768 blocks per pair)."""
    lib = H.get_lib()
    g = _gen_struct(H)
    d3 = _dims(1024, 1024, 1024)
    assert lib.hyenand_generate_kernel_spectrum(FAKE, ctypes.byref(g), FAKE, 8, 8192, 3, d3, 0, FAKE, 1 << 40,
                                                None) == 2
