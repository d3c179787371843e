"""Python binding of ``libhyenand.so``, the MI355X gated N-D FFT convolution.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the current HIP stream.  The
library must be built (``dimensional_fft_long_amd.build.build()``); the first
call raises if it is missing.

The operation (explainer "Native multi-dimensional subquadratic operators via
input-dependent long convolutions", section "HyenaND: native-space implicit
global kernel", output equation y[i]; gist.science summary, "Methodology",
"Boundary handling")::

    y[b,c,i] = sum_j sigmoid(alpha_c x[b,c,j] + beta_c) x[b,c,j] K_c[i-j]

zero outside the grid.  Entry points mirror ``include/hyenand.h``:

* ``kernel_spectrum(K, dims)``        -> K_hat (once per parameter set)
* ``fftconv_fwd(x, alpha, beta, K_hat)`` -> y
* ``fftconv_bwd(x, alpha, beta, K_hat, dy)`` -> (dx, dalpha, dbeta, dK): the
  backward, recomputing the forward transforms (explainer, "Implementation and
  operation patterns", "Concrete implementation pattern (PyTorch)")
* ``gated_fftconv`` / ``GatedFFTConvFunction`` -- the differentiable operation
  (torch autograd over the forward and the backward)
* ``fftconv_fwd_per_sample(x, alpha, beta, K_hat)`` -- input-dependent kernels:
  K_hat = kernel_spectrum(K) of kernels [B, C, *(2n-1)], one per (b, c);
  ``fftconv_bwd_per_sample(...)`` its backward (dK per (b, c))
* ``kernel_spectrum_circ(K)`` / ``fftconv_fwd_circ(...)`` /
  ``fftconv_bwd_circ(...)`` -- the circular mode (gist.science summary,
  "Boundary handling": periodic grids, no padding; K is [C, *dims] indexed by
  offset mod n)
* ``generate_kernel_spectrum(x, gen)`` / ``fftconv_fwd_generated(...)`` -- the
  input-dependent kernels generated on the GPU from x, alone or ahead of the
  forward in one call
* ``fftconv_fwd_noalloc(...)`` -- the forward with the library's static
  workspace (for callers that cannot allocate)

Calls without a ``workspace`` argument take one from a cache keyed by kind,
device, size and stream; ``release_workspaces()`` frees it.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhyenand.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1

EXPORTS = ("hyenand_status_string", "hyenand_version", "hyenand_kernel_spectrum_bytes",
           "hyenand_kernel_spectrum_tile", "hyenand_kernel_spectrum",
           "hyenand_fftconv_workspace_bytes", "hyenand_fftconv_workspace_min_bytes", "hyenand_fftconv_fwd",
           "hyenand_fftconv_fwd_traced", "hyenand_fftconv_launch_plan", "hyenand_fftconv_bwd",
           "hyenand_fftconv_bwd_workspace_bytes", "hyenand_fftconv_bwd_workspace_min_bytes",
           "hyenand_fftconv_bwd_traced", "hyenand_kernel_spectrum_circ_bytes", "hyenand_kernel_spectrum_circ_tile",
           "hyenand_kernel_spectrum_circ", "hyenand_fftconv_circ_workspace_bytes",
           "hyenand_fftconv_circ_workspace_min_bytes", "hyenand_fftconv_fwd_circ", "hyenand_fftconv_fwd_circ_traced",
           "hyenand_fftconv_fwd_per_sample", "hyenand_fftconv_fwd_per_sample_traced", "hyenand_fftconv_bwd_circ",
           "hyenand_fftconv_bwd_circ_workspace_bytes", "hyenand_fftconv_bwd_circ_workspace_min_bytes",
           "hyenand_fftconv_bwd_circ_traced", "hyenand_fftconv_bwd_per_sample",
           "hyenand_fftconv_bwd_per_sample_traced", "hyenand_generate_workspace_bytes",
           "hyenand_generate_kernel_spectrum", "hyenand_fftconv_fwd_noalloc",
           "hyenand_fftconv_fwd_noalloc_max_workspace", "hyenand_fftconv_fwd_generated",
           "hyenand_fftconv_fwd_generated_workspace_bytes", "hyenand_fftconv_fwd_generated_workspace_min_bytes")

_lib = None


class _Generator(ctypes.Structure):
    """hyenand_generator (include/hyenand.h): device pointers of the
    input-dependent kernel generator's parameters."""
    _fields_ = [("R", ctypes.c_int), ("D", ctypes.c_int)] + \
               [(k, ctypes.c_void_p) for k in ("Wreg", "breg", "q", "Wgam", "Wbet", "W1", "b1", "W2", "b2", "sigma")] + \
               [("omega0", ctypes.c_float)]


def get_lib() -> ctypes.CDLL:
    """Load ``libhyenand.so`` (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run dimensional_fft_long_amd.build.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.hyenand_status_string.argtypes = [I]
    lib.hyenand_status_string.restype = ctypes.c_char_p
    lib.hyenand_version.argtypes = []
    lib.hyenand_version.restype = I
    lib.hyenand_kernel_spectrum_bytes.argtypes = [I, I, P]
    lib.hyenand_kernel_spectrum_bytes.restype = SZ
    lib.hyenand_kernel_spectrum_tile.argtypes = [I, P]
    lib.hyenand_kernel_spectrum_tile.restype = I
    lib.hyenand_kernel_spectrum.argtypes = [P, P, I, I, P, P]
    lib.hyenand_kernel_spectrum.restype = I
    lib.hyenand_fftconv_workspace_bytes.argtypes = [I, I, I, P, I]
    lib.hyenand_fftconv_workspace_bytes.restype = SZ
    lib.hyenand_fftconv_workspace_min_bytes.argtypes = [I, I, I, P, I]
    lib.hyenand_fftconv_workspace_min_bytes.restype = SZ
    lib.hyenand_fftconv_fwd.argtypes = [P, P, P, P, P, I, I, I, P, I, P, SZ, P]
    lib.hyenand_fftconv_fwd.restype = I
    lib.hyenand_fftconv_fwd_traced.argtypes = [P, P, P, P, P, I, I, I, P, I, P, SZ, P, P, I, ctypes.POINTER(I)]
    lib.hyenand_fftconv_fwd_traced.restype = I
    lib.hyenand_fftconv_launch_plan.argtypes = [I, I, I, P, I, SZ, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.hyenand_fftconv_launch_plan.restype = I
    lib.hyenand_fftconv_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, P, I, P, SZ, P]
    lib.hyenand_fftconv_bwd.restype = I
    lib.hyenand_fftconv_bwd_traced.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, P, I, P, SZ, P, P, I,
                                               ctypes.POINTER(I)]
    lib.hyenand_fftconv_bwd_traced.restype = I
    lib.hyenand_fftconv_bwd_workspace_bytes.argtypes = [I, I, I, P, I, I]
    lib.hyenand_fftconv_bwd_workspace_bytes.restype = SZ
    lib.hyenand_fftconv_bwd_workspace_min_bytes.argtypes = [I, I, I, P, I, I]
    lib.hyenand_fftconv_bwd_workspace_min_bytes.restype = SZ
    lib.hyenand_fftconv_bwd_circ.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, P, I, P, SZ, P]
    lib.hyenand_fftconv_bwd_circ.restype = I
    lib.hyenand_fftconv_bwd_circ_traced.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, P, I, P, SZ, P, P, I,
                                                    ctypes.POINTER(I)]
    lib.hyenand_fftconv_bwd_circ_traced.restype = I
    lib.hyenand_fftconv_bwd_per_sample.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, P, I, P, SZ, P]
    lib.hyenand_fftconv_bwd_per_sample.restype = I
    lib.hyenand_fftconv_bwd_per_sample_traced.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, P, I, P, SZ, P, P,
                                                          I, ctypes.POINTER(I)]
    lib.hyenand_fftconv_bwd_per_sample_traced.restype = I
    lib.hyenand_fftconv_bwd_circ_workspace_bytes.argtypes = [I, I, I, P, I, I]
    lib.hyenand_fftconv_bwd_circ_workspace_bytes.restype = SZ
    lib.hyenand_fftconv_bwd_circ_workspace_min_bytes.argtypes = [I, I, I, P, I, I]
    lib.hyenand_fftconv_bwd_circ_workspace_min_bytes.restype = SZ
    lib.hyenand_kernel_spectrum_circ_bytes.argtypes = [I, I, P]
    lib.hyenand_kernel_spectrum_circ_bytes.restype = SZ
    lib.hyenand_kernel_spectrum_circ_tile.argtypes = [I, P]
    lib.hyenand_kernel_spectrum_circ_tile.restype = I
    lib.hyenand_kernel_spectrum_circ.argtypes = [P, P, I, I, P, P]
    lib.hyenand_kernel_spectrum_circ.restype = I
    lib.hyenand_fftconv_circ_workspace_bytes.argtypes = [I, I, I, P, I]
    lib.hyenand_fftconv_circ_workspace_bytes.restype = SZ
    lib.hyenand_fftconv_circ_workspace_min_bytes.argtypes = [I, I, I, P, I]
    lib.hyenand_fftconv_circ_workspace_min_bytes.restype = SZ
    lib.hyenand_fftconv_fwd_circ.argtypes = [P, P, P, P, P, I, I, I, P, I, P, SZ, P]
    lib.hyenand_fftconv_fwd_circ.restype = I
    lib.hyenand_fftconv_fwd_circ_traced.argtypes = [P, P, P, P, P, I, I, I, P, I, P, SZ, P, P, I, ctypes.POINTER(I)]
    lib.hyenand_fftconv_fwd_circ_traced.restype = I
    lib.hyenand_fftconv_fwd_per_sample.argtypes = [P, P, P, P, P, I, I, I, P, I, P, SZ, P]
    lib.hyenand_fftconv_fwd_per_sample.restype = I
    lib.hyenand_fftconv_fwd_per_sample_traced.argtypes = [P, P, P, P, P, I, I, I, P, I, P, SZ, P, P, I,
                                                          ctypes.POINTER(I)]
    lib.hyenand_fftconv_fwd_per_sample_traced.restype = I
    lib.hyenand_fftconv_fwd_noalloc.argtypes = [P, P, P, P, P, I, I, I, P, I, P]
    lib.hyenand_fftconv_fwd_noalloc.restype = I
    lib.hyenand_fftconv_fwd_noalloc_max_workspace.argtypes = []
    lib.hyenand_fftconv_fwd_noalloc_max_workspace.restype = SZ
    lib.hyenand_generate_workspace_bytes.argtypes = [I, I, I, P]
    lib.hyenand_generate_workspace_bytes.restype = SZ
    lib.hyenand_generate_kernel_spectrum.argtypes = [P, ctypes.POINTER(_Generator), P, I, I, I, P, I, P, SZ, P]
    lib.hyenand_generate_kernel_spectrum.restype = I
    lib.hyenand_fftconv_fwd_generated.argtypes = [P, P, P, ctypes.POINTER(_Generator), P, P, I, I, I, P, I, P, SZ, P]
    lib.hyenand_fftconv_fwd_generated.restype = I
    lib.hyenand_fftconv_fwd_generated_workspace_bytes.argtypes = [I, I, I, P, I]
    lib.hyenand_fftconv_fwd_generated_workspace_bytes.restype = SZ
    lib.hyenand_fftconv_fwd_generated_workspace_min_bytes.argtypes = [I, I, I, P, I]
    lib.hyenand_fftconv_fwd_generated_workspace_min_bytes.restype = SZ
    _lib = lib
    return lib


_P = ctypes.c_void_p


class HyenandError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {get_lib().hyenand_status_string(code).decode()} ({code})")
        self.code = code


def _dims_arr(dims):
    arr = (ctypes.c_int64 * len(dims))(*[int(v) for v in dims])
    return arr


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"x must be float32 or bfloat16, got {t}")


def spectrum_bytes(C: int, dims) -> int:
    return int(get_lib().hyenand_kernel_spectrum_bytes(C, len(dims), _dims_arr(dims)))


def spectrum_tile(dims) -> int:
    """Slot tile T of the K_hat layout (see hyenand_kernel_spectrum_bytes)."""
    return int(get_lib().hyenand_kernel_spectrum_tile(len(dims), _dims_arr(dims)))


def workspace_bytes(B: int, C: int, dims, dtype=torch.float32, minimum: bool = False) -> int:
    lib = get_lib()
    f = lib.hyenand_fftconv_workspace_min_bytes if minimum else lib.hyenand_fftconv_workspace_bytes
    return int(f(B, C, len(dims), _dims_arr(dims), _dtype_code(dtype)))


def _ws_bytes(workspace, device) -> int:
    """A caller's workspace: a contiguous tensor on ``device`` (the kernels
    write it as device memory); its size in bytes."""
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch tensor")
    if workspace.device != torch.device(device) or not workspace.is_contiguous():
        raise TypeError(f"workspace must be a contiguous tensor on {device}")
    return workspace.numel() * workspace.element_size()


def _check_spectrum_out(out, nbytes, device):
    if not isinstance(out, torch.Tensor) or out.dtype != torch.complex64:
        raise TypeError("out must be a complex64 tensor")
    if out.device != torch.device(device) or not out.is_contiguous():
        raise TypeError(f"out must be a contiguous tensor on {device}")
    if out.numel() * 8 < nbytes:
        raise ValueError(f"out holds {out.numel() * 8} bytes, the spectrum needs {nbytes}")


def kernel_spectrum(K: torch.Tensor, dims=None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """K: fp32 device tensor [C, 2n_0-1, ..., 2n_{d-1}-1] -> K_hat (complex64 flat [C, ksz])."""
    if dims is None:
        dims = tuple((s + 1) // 2 for s in K.shape[1:])
    dims = tuple(int(v) for v in dims)
    C = int(K.shape[0])
    if K.dtype != torch.float32 or not K.is_cuda or not K.is_contiguous():
        raise TypeError("K must be a contiguous float32 device tensor")
    if tuple(K.shape[1:]) != tuple(2 * n - 1 for n in dims):
        raise ValueError("K must be [C, 2n-1, ...]")
    nbytes = spectrum_bytes(C, dims)
    if nbytes == 0 and C > 0:
        raise HyenandError(ERR_UNSUPPORTED, "kernel_spectrum")
    if out is None:
        out = torch.empty(nbytes // 8, dtype=torch.complex64, device=K.device).view(C, -1) if C else \
            torch.empty(0, dtype=torch.complex64, device=K.device)
    else:
        _check_spectrum_out(out, nbytes, K.device)
    rc = get_lib().hyenand_kernel_spectrum(_P(K.data_ptr()), _P(out.data_ptr()), C, len(dims), _dims_arr(dims),
                                     _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "kernel_spectrum")
    return out


_ws_cache: dict = {}


def _cached_ws(kind: str, nbytes: int, device, stream):
    """A workspace of ``nbytes`` sized once per shape and reused (explainer,
    "Implementation and operation patterns", "Memory allocation and buffer
    management": the size follows from the input shape).  One buffer per
    (kind, device, size, stream): calls in flight on different streams never
    share a workspace, and calls on one stream are ordered by the stream."""
    st = torch.cuda.current_stream(device) if stream is None else stream
    key = (kind, str(device), int(nbytes), int(st.cuda_stream))
    buf = _ws_cache.get(key)
    if buf is None:
        buf = torch.empty(max(int(nbytes), 8), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf, int(nbytes)


def release_workspaces() -> None:
    """Free the workspaces the calls above cached (one per shape and stream;
    a long-running program that meets many shapes calls this now and then).
    Each buffer's device is synchronised first, so no call in flight still
    uses it; the next call allocates afresh."""
    for dev in {buf.device for buf in _ws_cache.values()}:
        torch.cuda.synchronize(dev)
    _ws_cache.clear()


def _workspace(B, C, dims, dtype, device, stream=None):
    return _cached_ws("fwd", workspace_bytes(B, C, dims, dtype), device, stream)


def _check_out(t, name, shape, dtype, device, like=None):
    """A caller-provided output: contiguous, on ``device``, of exactly ``shape``
    and ``dtype``, and not overlapping ``like`` (the input it must not alias)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != torch.device(device) or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous tensor on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if like is not None and t.numel() > 0:
        a0, a1 = t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()
        b0, b1 = like.data_ptr(), like.data_ptr() + like.numel() * like.element_size()
        if a0 < b1 and b0 < a1:
            raise ValueError(f"{name} must not overlap the input")
    return t


def fftconv_fwd(x: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor, K_hat: torch.Tensor,
                y: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Gated N-D linear convolution; x [B, C, *dims] fp32 or bf16 on the device."""
    if not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous device tensor")
    dt = _dtype_code(x.dtype)
    B, C = int(x.shape[0]), int(x.shape[1])
    dims = tuple(int(v) for v in x.shape[2:])
    for t, nm in ((alpha, "alpha"), (beta, "beta")):
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous() or t.numel() != C:
            raise TypeError(f"{nm} must be a contiguous float32 tensor of C elements on {x.device}")
    if K_hat.dtype != torch.complex64 or K_hat.device != x.device or not K_hat.is_contiguous():
        raise TypeError("K_hat must be the contiguous complex64 output of kernel_spectrum")
    if K_hat.numel() * 8 < spectrum_bytes(C, dims):
        raise ValueError("K_hat is smaller than the spectrum of this shape")
    y = torch.empty_like(x) if y is None else _check_out(y, "y", x.shape, x.dtype, x.device, like=x)
    if workspace is None:
        workspace, ws_bytes = _workspace(B, C, dims, x.dtype, x.device, stream)
    else:
        ws_bytes = _ws_bytes(workspace, x.device)
    rc = get_lib().hyenand_fftconv_fwd(_P(x.data_ptr()), _P(alpha.data_ptr()), _P(beta.data_ptr()), _P(K_hat.data_ptr()),
                                 _P(y.data_ptr()), B, C, len(dims), _dims_arr(dims), dt,
                                 _P(workspace.data_ptr()), ws_bytes, _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "fftconv_fwd")
    return y


def launch_plan(B: int, C: int, dims, dtype, workspace_bytes: int) -> dict:
    """How a forward call with this workspace runs: kernel launches and channels per chunk."""
    n, ch = ctypes.c_int(0), ctypes.c_int(0)
    rc = get_lib().hyenand_fftconv_launch_plan(B, C, len(dims), _dims_arr(dims), _dtype_code(dtype),
                                               int(workspace_bytes), ctypes.byref(n), ctypes.byref(ch))
    if rc != OK:
        raise HyenandError(rc, "launch_plan")
    return {"launches": n.value, "chunk_channels": ch.value}


PASS_NAMES = {1: ("conv1d",), 2: ("row_fwd", "col_out", "row_inv"),
              3: ("row_fwd", "col_mid_fwd", "col_out", "col_mid_inv", "row_inv")}


def uses_fused2d(dims, circular: bool = False) -> bool:
    """True when the forward runs the on-chip 2-D kernel (one launch, no
    workspace): zero-padded 2-D grids with both extents in [4, 64]."""
    return (not circular and len(dims) == 2 and all(4 <= int(n) <= 64 for n in dims)
            and all(int(n) & (int(n) - 1) == 0 for n in dims))


def pass_names(dims, circular: bool = False):
    """Names of the kernels one channel chunk of a forward call launches, in order."""
    if uses_fused2d(dims, circular):
        return ("fused2d",)
    return PASS_NAMES[len(dims)]


def fftconv_fwd_traced(x, alpha, beta, K_hat, y, workspace, events, stream=None) -> int:
    """fftconv_fwd recording ``events`` (torch.cuda.Event list, timing enabled)
    before each kernel launch and after the last; returns the launch count."""
    B, C = int(x.shape[0]), int(x.shape[1])
    dims = tuple(int(v) for v in x.shape[2:])
    st = torch.cuda.current_stream() if stream is None else stream
    for e in events:
        if e.cuda_event == 0:     # torch creates the HIP event on its first record
            e.record(st)
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    n = ctypes.c_int(0)
    ws_bytes = _ws_bytes(workspace, x.device)
    rc = get_lib().hyenand_fftconv_fwd_traced(
        _P(x.data_ptr()), _P(alpha.data_ptr()), _P(beta.data_ptr()), _P(K_hat.data_ptr()), _P(y.data_ptr()),
        B, C, len(dims), _dims_arr(dims), _dtype_code(x.dtype), _P(workspace.data_ptr()), ws_bytes,
        _stream(stream), arr, len(events), ctypes.byref(n))
    if rc != OK:
        raise HyenandError(rc, "fftconv_fwd_traced")
    return int(n.value)


def bwd_workspace_bytes(B: int, C: int, dims, dtype=torch.float32, with_dK: bool = True,
                        minimum: bool = False, circular: bool = False) -> int:
    lib = get_lib()
    if circular:
        f = (lib.hyenand_fftconv_bwd_circ_workspace_min_bytes if minimum
             else lib.hyenand_fftconv_bwd_circ_workspace_bytes)
    else:
        f = lib.hyenand_fftconv_bwd_workspace_min_bytes if minimum else lib.hyenand_fftconv_bwd_workspace_bytes
    return int(f(B, C, len(dims), _dims_arr(dims), _dtype_code(dtype), int(bool(with_dK))))


def _bwd_workspace(B, C, dims, dtype, with_dK, device, circular=False, stream=None):
    return _cached_ws("bwd", bwd_workspace_bytes(B, C, dims, dtype, with_dK, circular=circular), device, stream)


def _bwd_args(x, alpha, beta, K_hat, dy, dx, dalpha, dbeta, dK, with_dK, workspace, circular=False,
              per_sample=False, stream=None):
    if not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous device tensor")
    if dy.shape != x.shape or dy.dtype != x.dtype or dy.device != x.device or not dy.is_contiguous():
        raise TypeError("dy must be a contiguous device tensor with the shape and dtype of x")
    B, C = int(x.shape[0]), int(x.shape[1])
    dims = tuple(int(v) for v in x.shape[2:])
    for t, nm in ((alpha, "alpha"), (beta, "beta")):
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous() or t.numel() != C:
            raise TypeError(f"{nm} must be a contiguous float32 tensor of C elements on {x.device}")
    if K_hat.dtype != torch.complex64 or K_hat.device != x.device or not K_hat.is_contiguous():
        raise TypeError("K_hat must be the contiguous complex64 output of kernel_spectrum")
    need = spectrum_circ_bytes(C, dims) if circular else spectrum_bytes(C, dims) * (B if per_sample else 1)
    if K_hat.numel() * 8 < need:
        raise ValueError("K_hat is smaller than the spectrum of this shape")
    dev = x.device
    dx = torch.empty_like(x) if dx is None else _check_out(dx, "dx", x.shape, x.dtype, dev, like=x)
    if dx is not None:
        _check_out(dx, "dx", x.shape, x.dtype, dev, like=dy)
    dalpha = torch.empty(C, dtype=torch.float32, device=dev) if dalpha is None else \
        _check_out(dalpha, "dalpha", (C,), torch.float32, dev)
    dbeta = torch.empty(C, dtype=torch.float32, device=dev) if dbeta is None else \
        _check_out(dbeta, "dbeta", (C,), torch.float32, dev)
    kdims = dims if circular else tuple(2 * n - 1 for n in dims)
    kshape = ((B,) if per_sample else ()) + (C,) + kdims
    if with_dK and dK is None:
        dK = torch.empty(kshape, dtype=torch.float32, device=dev)
    elif dK is not None:
        _check_out(dK, "dK", kshape, torch.float32, dev)
    if workspace is None:
        workspace, ws_bytes = _bwd_workspace(1 if per_sample else B, C, dims, x.dtype, dK is not None, dev,
                                             circular, stream)
    else:
        ws_bytes = _ws_bytes(workspace, x.device)
    args = [_P(x.data_ptr()), _P(alpha.data_ptr()), _P(beta.data_ptr()), _P(K_hat.data_ptr()), _P(dy.data_ptr()),
            _P(dx.data_ptr()), _P(dalpha.data_ptr()), _P(dbeta.data_ptr()),
            _P(dK.data_ptr()) if dK is not None else None, B, C, len(dims), _dims_arr(dims),
            _dtype_code(x.dtype), _P(workspace.data_ptr()), ws_bytes]
    return args, (dx, dalpha, dbeta, dK)


def fftconv_bwd(x, alpha, beta, K_hat, dy, dx=None, dalpha=None, dbeta=None, dK=None, with_dK: bool = True,
                workspace=None, stream=None):
    """Backward of fftconv_fwd for the output gradient dy.

    Returns (dx [B, C, *dims] in x's dtype, dalpha [C], dbeta [C], dK [C, *(2*dims-1)] or None)."""
    args, outs = _bwd_args(x, alpha, beta, K_hat, dy, dx, dalpha, dbeta, dK, with_dK, workspace, stream=stream)
    rc = get_lib().hyenand_fftconv_bwd(*args, _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "fftconv_bwd")
    return outs


BWD_PASS_NAMES = {
    (1, False): ("conv1d_bwd", "gate_reduce"),
    (1, True): ("conv1d_bwd", "gate_reduce", "corr1d", "dk_row"),
    (2, False): ("row_fwd_dy", "col_out_bwd", "row_inv_bwd", "gate_reduce"),
    (2, True): ("row_fwd_dy", "row_fwd_u", "col_out_bwd", "row_inv_bwd", "gate_reduce", "dk_row"),
    (3, False): ("row_fwd_dy", "col_mid_fwd_dy", "col_out_bwd", "col_mid_inv", "row_inv_bwd", "gate_reduce"),
    (3, True): ("row_fwd_dy", "row_fwd_u", "col_mid_fwd_dy", "col_mid_fwd_u", "col_out_bwd", "col_mid_inv",
                "row_inv_bwd", "gate_reduce", "mid_inv_dk", "dk_row"),
    # 1-D signals longer than 1024 (four-step transforms)
    ("long", False): ("lng_col_fwd_dy", "lng_row_du", "lng_col_inv_bwd", "gate_reduce"),
    ("long", True): ("lng_col_fwd_dy", "lng_col_fwd_u", "lng_row_dk", "lng_row_du", "lng_col_inv_bwd", "gate_reduce",
                     "lng_col_dk"),
    # n > 2^21 (4096-point rows): the kernel-gradient row pass also writes du
    ("long4096", True): ("lng_col_fwd_dy", "lng_col_fwd_u", "lng_row_dk", "lng_col_inv_bwd", "gate_reduce",
                         "lng_col_dk"),
}


def fftconv_bwd_traced(x, alpha, beta, K_hat, dy, outs, workspace, events, stream=None, circular=False,
                       per_sample=False) -> int:
    """fftconv_bwd (fftconv_bwd_circ with ``circular``, fftconv_bwd_per_sample
    with ``per_sample``) into ``outs`` = (dx, dalpha, dbeta, dK or None),
    recording ``events`` before each kernel launch and after the last; returns
    the launch count."""
    dx, dalpha, dbeta, dK = outs
    args, _ = _bwd_args(x, alpha, beta, K_hat, dy, dx, dalpha, dbeta, dK, dK is not None, workspace, circular,
                        per_sample, stream)
    st = torch.cuda.current_stream() if stream is None else stream
    for e in events:
        if e.cuda_event == 0:
            e.record(st)
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    n = ctypes.c_int(0)
    lib = get_lib()
    f = (lib.hyenand_fftconv_bwd_circ_traced if circular else
         (lib.hyenand_fftconv_bwd_per_sample_traced if per_sample else lib.hyenand_fftconv_bwd_traced))
    rc = f(*args, _stream(stream), arr, len(events), ctypes.byref(n))
    if rc != OK:
        raise HyenandError(rc, "fftconv_bwd_traced")
    return int(n.value)


class GatedFFTConvFunction(torch.autograd.Function):
    """The library's forward and backward as one differentiable operation.

    Inputs: x [B, C, *dims] (fp32 or bf16), alpha and beta [C], and the
    spatial kernel K: [C, *(2n-1)] shared by the batch, [B, C, *(2n-1)] one per
    (b, c) (input-dependent kernels), or [C, *dims] with ``circular=True``.
    Only x, alpha, beta and the kernel spectrum are kept for the backward, which
    recomputes every transform from them: the recompute-instead-of-store
    trade-off the explainer recommends for the FFT intermediates ("Gradient
    flow and numerical stability", gradient checkpointing).  Gradients flow to
    x, alpha, beta and K; the FFT workspaces are sized once per shape and
    reused."""

    @staticmethod
    def forward(ctx, x, alpha, beta, K, circular=False):
        dims = tuple(int(v) for v in x.shape[2:])
        mode = "circular" if circular else ("per_sample" if K.dim() == x.dim() else "shared")
        if mode == "circular" and K.dim() == x.dim():
            raise ValueError("per-sample kernels are built for the zero-padded mode only")
        spec, fwd = {"circular": (kernel_spectrum_circ, fftconv_fwd_circ),
                     "per_sample": (kernel_spectrum_per_sample, fftconv_fwd_per_sample),
                     "shared": (lambda k: kernel_spectrum(k, dims), fftconv_fwd)}[mode]
        K_hat = spec(K.contiguous())
        ctx.mode = mode
        ctx.want_dK = bool(ctx.needs_input_grad[3])
        ctx.save_for_backward(x, alpha, beta, K_hat)
        return fwd(x, alpha, beta, K_hat)

    @staticmethod
    def backward(ctx, dy):
        x, alpha, beta, K_hat = ctx.saved_tensors
        bwd = {"circular": fftconv_bwd_circ, "per_sample": fftconv_bwd_per_sample, "shared": fftconv_bwd}[ctx.mode]
        dx, dalpha, dbeta, dK = bwd(x, alpha, beta, K_hat, dy.contiguous(), with_dK=ctx.want_dK)
        return dx, dalpha, dbeta, dK, None  # no gradient for the boundary flag


def gated_fftconv(x, alpha, beta, K, circular: bool = False) -> torch.Tensor:
    """Differentiable gated N-D convolution (GatedFFTConvFunction)."""
    return GatedFFTConvFunction.apply(x, alpha, beta, K, circular)


# ----------------------------------------------------------- circular mode

def fftconv_bwd_circ(x, alpha, beta, K_hat, dy, dx=None, dalpha=None, dbeta=None, dK=None, with_dK: bool = True,
                     workspace=None, stream=None):
    """Backward of fftconv_fwd_circ for the output gradient dy; K_hat from
    kernel_spectrum_circ.  Returns (dx, dalpha, dbeta, dK [C, *dims] or None),
    dK indexed by offset mod n like the circular K."""
    args, outs = _bwd_args(x, alpha, beta, K_hat, dy, dx, dalpha, dbeta, dK, with_dK, workspace, circular=True,
                           stream=stream)
    rc = get_lib().hyenand_fftconv_bwd_circ(*args, _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "fftconv_bwd_circ")
    return outs


def spectrum_circ_bytes(C: int, dims) -> int:
    return int(get_lib().hyenand_kernel_spectrum_circ_bytes(C, len(dims), _dims_arr(dims)))


def circ_workspace_bytes(B: int, C: int, dims, dtype=torch.float32, minimum: bool = False) -> int:
    lib = get_lib()
    f = lib.hyenand_fftconv_circ_workspace_min_bytes if minimum else lib.hyenand_fftconv_circ_workspace_bytes
    return int(f(B, C, len(dims), _dims_arr(dims), _dtype_code(dtype)))


def kernel_spectrum_circ(K: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Circular mode: K fp32 device tensor [C, *dims] (index = offset mod n) -> K_hat (complex64 [C, ksz])."""
    dims = tuple(int(v) for v in K.shape[1:])
    C = int(K.shape[0])
    if K.dtype != torch.float32 or not K.is_cuda or not K.is_contiguous():
        raise TypeError("K must be a contiguous float32 device tensor")
    nbytes = spectrum_circ_bytes(C, dims)
    if nbytes == 0 and C > 0:
        raise HyenandError(ERR_UNSUPPORTED, "kernel_spectrum_circ")
    if out is None:
        out = torch.empty(nbytes // 8, dtype=torch.complex64, device=K.device).view(C, -1) if C else \
            torch.empty(0, dtype=torch.complex64, device=K.device)
    else:
        _check_spectrum_out(out, nbytes, K.device)
    rc = get_lib().hyenand_kernel_spectrum_circ(_P(K.data_ptr()), _P(out.data_ptr()), C, len(dims), _dims_arr(dims),
                                                _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "kernel_spectrum_circ")
    return out


def _circ_args(x, alpha, beta, K_hat, y, workspace, stream=None):
    if not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous device tensor")
    B, C = int(x.shape[0]), int(x.shape[1])
    dims = tuple(int(v) for v in x.shape[2:])
    for t, nm in ((alpha, "alpha"), (beta, "beta")):
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous() or t.numel() != C:
            raise TypeError(f"{nm} must be a contiguous float32 tensor of C elements on {x.device}")
    if K_hat.dtype != torch.complex64 or K_hat.device != x.device or not K_hat.is_contiguous():
        raise TypeError("K_hat must be the contiguous complex64 output of kernel_spectrum_circ")
    if K_hat.numel() * 8 < spectrum_circ_bytes(C, dims):
        raise ValueError("K_hat is smaller than the circular spectrum of this shape")
    y = torch.empty_like(x) if y is None else _check_out(y, "y", x.shape, x.dtype, x.device, like=x)
    if workspace is None:
        workspace, ws_bytes = _cached_ws("circ", circ_workspace_bytes(B, C, dims, x.dtype), x.device, stream)
    else:
        ws_bytes = _ws_bytes(workspace, x.device)
    args = [_P(x.data_ptr()), _P(alpha.data_ptr()), _P(beta.data_ptr()), _P(K_hat.data_ptr()), _P(y.data_ptr()),
            B, C, len(dims), _dims_arr(dims), _dtype_code(x.dtype), _P(workspace.data_ptr()), ws_bytes]
    return args, y


def fftconv_fwd_circ(x, alpha, beta, K_hat, y=None, workspace=None, stream=None) -> torch.Tensor:
    """Circular-mode gated N-D convolution (periodic grid, no padding); K_hat from kernel_spectrum_circ."""
    args, y = _circ_args(x, alpha, beta, K_hat, y, workspace, stream)
    rc = get_lib().hyenand_fftconv_fwd_circ(*args, _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "fftconv_fwd_circ")
    return y


def fftconv_fwd_circ_traced(x, alpha, beta, K_hat, y, workspace, events, stream=None) -> int:
    """fftconv_fwd_circ recording ``events`` before each kernel launch and after the last."""
    args, y = _circ_args(x, alpha, beta, K_hat, y, workspace, stream)
    st = torch.cuda.current_stream() if stream is None else stream
    for e in events:
        if e.cuda_event == 0:
            e.record(st)
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    n = ctypes.c_int(0)
    rc = get_lib().hyenand_fftconv_fwd_circ_traced(*args, _stream(stream), arr, len(events), ctypes.byref(n))
    if rc != OK:
        raise HyenandError(rc, "fftconv_fwd_circ_traced")
    return int(n.value)


# ------------------------------------------------------- per-sample kernels

def kernel_spectrum_per_sample(K: torch.Tensor, stream=None) -> torch.Tensor:
    """Input-dependent kernels K [B, C, *(2n-1)] (fp32, device) -> K_hat [B * C, ksz]."""
    B, C = int(K.shape[0]), int(K.shape[1])
    dims = tuple((v + 1) // 2 for v in K.shape[2:])
    return kernel_spectrum(K.reshape((B * C,) + tuple(K.shape[2:])), dims, stream=stream)


def _ps_args(x, alpha, beta, K_hat, y, workspace, stream=None):
    if not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous device tensor")
    B, C = int(x.shape[0]), int(x.shape[1])
    dims = tuple(int(v) for v in x.shape[2:])
    for t, nm in ((alpha, "alpha"), (beta, "beta")):
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous() or t.numel() != C:
            raise TypeError(f"{nm} must be a contiguous float32 tensor of C elements on {x.device}")
    if K_hat.dtype != torch.complex64 or K_hat.device != x.device or not K_hat.is_contiguous():
        raise TypeError("K_hat must be the contiguous complex64 output of kernel_spectrum_per_sample")
    if K_hat.numel() * 8 < spectrum_bytes(B * C, dims):
        raise ValueError("K_hat must hold B * C spectra of this shape")
    y = torch.empty_like(x) if y is None else _check_out(y, "y", x.shape, x.dtype, x.device, like=x)
    if workspace is None:
        workspace, ws_bytes = _workspace(B, C, dims, x.dtype, x.device, stream)
    else:
        ws_bytes = _ws_bytes(workspace, x.device)
    return [_P(x.data_ptr()), _P(alpha.data_ptr()), _P(beta.data_ptr()), _P(K_hat.data_ptr()), _P(y.data_ptr()),
            B, C, len(dims), _dims_arr(dims), _dtype_code(x.dtype), _P(workspace.data_ptr()), ws_bytes], y


def fftconv_fwd_per_sample(x, alpha, beta, K_hat, y=None, workspace=None, stream=None) -> torch.Tensor:
    """Gated N-D convolution with one kernel per (b, c) (K_hat from kernel_spectrum_per_sample)."""
    args, y = _ps_args(x, alpha, beta, K_hat, y, workspace, stream)
    rc = get_lib().hyenand_fftconv_fwd_per_sample(*args, _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "fftconv_fwd_per_sample")
    return y


def fftconv_bwd_per_sample(x, alpha, beta, K_hat, dy, dx=None, dalpha=None, dbeta=None, dK=None,
                           with_dK: bool = True, workspace=None, stream=None):
    """Backward of fftconv_fwd_per_sample for the output gradient dy; K_hat from
    kernel_spectrum_per_sample.  Returns (dx, dalpha [C], dbeta [C],
    dK [B, C, *(2*dims-1)] or None): one kernel gradient per (b, c).  The
    workspace is that of a batch of one (bwd_workspace_bytes(1, C, dims))."""
    args, outs = _bwd_args(x, alpha, beta, K_hat, dy, dx, dalpha, dbeta, dK, with_dK, workspace, per_sample=True,
                           stream=stream)
    rc = get_lib().hyenand_fftconv_bwd_per_sample(*args, _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "fftconv_bwd_per_sample")
    return outs


def fftconv_fwd_per_sample_traced(x, alpha, beta, K_hat, y, workspace, events, stream=None) -> int:
    args, y = _ps_args(x, alpha, beta, K_hat, y, workspace, stream)
    st = torch.cuda.current_stream() if stream is None else stream
    for e in events:
        if e.cuda_event == 0:
            e.record(st)
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    n = ctypes.c_int(0)
    rc = get_lib().hyenand_fftconv_fwd_per_sample_traced(*args, _stream(stream), arr, len(events), ctypes.byref(n))
    if rc != OK:
        raise HyenandError(rc, "fftconv_fwd_per_sample_traced")
    return int(n.value)


# --------------------------------------------------- allocation-free forward

def noalloc_max_workspace() -> int:
    """Bytes of the static device scratch behind fftconv_fwd_noalloc."""
    return int(get_lib().hyenand_fftconv_fwd_noalloc_max_workspace())


def fftconv_fwd_noalloc(x, alpha, beta, K_hat, y, stream=None) -> torch.Tensor:
    """fftconv_fwd through the allocation-free entry point: the library's static
    device scratch serves as the workspace; the caller provides y.  Calls that
    overlap in time on one GPU share that scratch and race."""
    if not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous device tensor")
    B, C = int(x.shape[0]), int(x.shape[1])
    dims = tuple(int(v) for v in x.shape[2:])
    for t, nm in ((alpha, "alpha"), (beta, "beta")):
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous() or t.numel() != C:
            raise TypeError(f"{nm} must be a contiguous float32 tensor of C elements on {x.device}")
    if K_hat.dtype != torch.complex64 or K_hat.device != x.device or not K_hat.is_contiguous():
        raise TypeError("K_hat must be the contiguous complex64 output of kernel_spectrum")
    if K_hat.numel() * 8 < spectrum_bytes(C, dims):
        raise ValueError("K_hat is smaller than the spectrum of this shape")
    _check_out(y, "y", x.shape, x.dtype, x.device, like=x)
    rc = get_lib().hyenand_fftconv_fwd_noalloc(_P(x.data_ptr()), _P(alpha.data_ptr()), _P(beta.data_ptr()),
                                               _P(K_hat.data_ptr()), _P(y.data_ptr()), B, C, len(dims),
                                               _dims_arr(dims), _dtype_code(x.dtype), _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "fftconv_fwd_noalloc")
    return y


# ------------------------------------------------ generated per-sample kernels

GEN_KEYS = ("Wreg", "breg", "q", "Wgam", "Wbet", "W1", "b1", "W2", "b2", "sigma")


def generate_workspace_bytes(B: int, C: int, dims) -> int:
    return int(get_lib().hyenand_generate_workspace_bytes(B, C, len(dims), _dims_arr(dims)))


def _gen_struct(x: torch.Tensor, gen: dict):
    """Checks the generator parameters against x; returns the hyenand_generator."""
    if not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous device tensor")
    C = int(x.shape[1])
    d = x.dim() - 2
    shapes = {"breg": None, "q": None, "Wgam": None, "Wbet": None, "W1": (16, d), "b1": (16,), "W2": (C, 16),
              "b2": (C,), "sigma": (C,)}
    for k in GEN_KEYS:
        t = gen[k]
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous():
            raise TypeError(f"generator parameter {k} must be a contiguous float32 tensor on {x.device}")
        if shapes.get(k) is not None and tuple(t.shape) != shapes[k]:
            raise ValueError(f"generator parameter {k} must have shape {shapes[k]}")
    R, D = int(gen["Wreg"].shape[0]), int(gen["Wreg"].shape[1])
    want = {"Wreg": (R, D, C), "breg": (R, D), "q": (D,), "Wgam": (16, D), "Wbet": (16, D)}
    for k, shp in want.items():
        if tuple(gen[k].shape) != shp:
            raise ValueError(f"generator parameter {k} must have shape {shp}")
    return _Generator(R, D, *[gen[k].data_ptr() for k in GEN_KEYS], float(gen["omega0"]))


def generate_kernel_spectrum(x: torch.Tensor, gen: dict, out: torch.Tensor | None = None, workspace=None,
                             stream=None) -> torch.Tensor:
    """Spectra of the input-dependent kernels of x (registers -> softmax
    control -> FiLM-modulated SIREN -> Gaussian window, hyenand.h), one per
    (b, c), generated on the GPU without forming the kernels: K_hat [B * C, ksz]
    for fftconv_fwd_per_sample / fftconv_bwd_per_sample.  ``gen``: fp32 device
    tensors Wreg [R, D, C], breg [R, D], q [D], Wgam [16, D], Wbet [16, D],
    W1 [16, d], b1 [16], W2 [C, 16], b2 [C], sigma [C], and omega0 (float)."""
    g = _gen_struct(x, gen)
    B, C = int(x.shape[0]), int(x.shape[1])
    dims = tuple(int(v) for v in x.shape[2:])
    d = len(dims)
    nbytes = spectrum_bytes(B * C, dims)
    if nbytes == 0:
        raise HyenandError(ERR_UNSUPPORTED, "generate_kernel_spectrum")
    if out is None:
        out = torch.empty(nbytes // 8, dtype=torch.complex64, device=x.device).view(B * C, -1)
    else:
        _check_spectrum_out(out, nbytes, x.device)
    if workspace is None:
        workspace, ws_bytes = _cached_ws("gen", generate_workspace_bytes(B, C, dims), x.device, stream)
    else:
        ws_bytes = _ws_bytes(workspace, x.device)
    rc = get_lib().hyenand_generate_kernel_spectrum(_P(x.data_ptr()), ctypes.byref(g), _P(out.data_ptr()), B, C, d,
                                                    _dims_arr(dims), _dtype_code(x.dtype), _P(workspace.data_ptr()),
                                                    ws_bytes, _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "generate_kernel_spectrum")
    return out


def generated_workspace_bytes(B: int, C: int, dims, dtype=torch.float32, minimum: bool = False) -> int:
    f = (get_lib().hyenand_fftconv_fwd_generated_workspace_min_bytes if minimum
         else get_lib().hyenand_fftconv_fwd_generated_workspace_bytes)
    return int(f(B, C, len(dims), _dims_arr(dims), _dtype_code(dtype)))


def fftconv_fwd_generated(x: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor, gen: dict,
                          K_hat: torch.Tensor | None = None, y: torch.Tensor | None = None, workspace=None,
                          stream=None):
    """Forward with the input-dependent kernels of x generated in the same call
    (the generator's spectra, then the forward chains; hyenand.h).
    Returns (y, K_hat [B * C, ksz]); K_hat feeds fftconv_bwd_per_sample."""
    g = _gen_struct(x, gen)
    B, C = int(x.shape[0]), int(x.shape[1])
    dims = tuple(int(v) for v in x.shape[2:])
    for t, nm in ((alpha, "alpha"), (beta, "beta")):
        if t.dtype != torch.float32 or t.device != x.device or not t.is_contiguous() or t.numel() != C:
            raise TypeError(f"{nm} must be a contiguous float32 tensor of C elements on {x.device}")
    nbytes = spectrum_bytes(B * C, dims)
    if nbytes == 0:
        raise HyenandError(ERR_UNSUPPORTED, "fftconv_fwd_generated")
    if K_hat is None:
        K_hat = torch.empty(nbytes // 8, dtype=torch.complex64, device=x.device).view(B * C, -1)
    else:
        _check_spectrum_out(K_hat, nbytes, x.device)
    y = torch.empty_like(x) if y is None else _check_out(y, "y", x.shape, x.dtype, x.device, like=x)
    if workspace is None:
        workspace, ws_bytes = _cached_ws("gen_fwd", generated_workspace_bytes(B, C, dims, x.dtype), x.device, stream)
    else:
        ws_bytes = _ws_bytes(workspace, x.device)
    rc = get_lib().hyenand_fftconv_fwd_generated(_P(x.data_ptr()), _P(alpha.data_ptr()), _P(beta.data_ptr()),
                                                 ctypes.byref(g), _P(K_hat.data_ptr()), _P(y.data_ptr()), B, C,
                                                 len(dims), _dims_arr(dims), _dtype_code(x.dtype),
                                                 _P(workspace.data_ptr()), ws_bytes, _stream(stream))
    if rc != OK:
        raise HyenandError(rc, "fftconv_fwd_generated")
    return y, K_hat
