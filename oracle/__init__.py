"""Oracle: plain fp64 CPU reference for HyenaND's gated N-D linear convolution.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library ``dimensional_fft_long_amd`` and never imports it.

What it computes (explainer "Native multi-dimensional subquadratic operators via
input-dependent long convolutions", section "HyenaND: native-space implicit
global kernel", output equation for y[i]; gist.science summary of the same
paper, section "Methodology", item "Boundary handling")::

    y[b,c,i] = sum_j phi_c(x[b,c,j]) * x[b,c,j] * K_c[i-j],   i, j in the grid,
    phi_c(v) = 1 / (1 + exp(-(alpha_c v + beta_c))),

zero outside the grid (non-circular), K_c on offsets [-(n-1), n-1] per axis with
offset 0 at index n-1, one kernel per channel shared over the batch.

Routes (all fp64, in ``oracle.c``):
  * ``direct``        -- O1, the sum written out, every output.
  * ``direct_points`` -- O1 at chosen outputs (for grids too big for O2).
  * ``fftconv``       -- O2, explicit zero padding to 2n, textbook radix-2 FFT.
  * ``kernel_spectrum`` -- the full DFT of the wrap-placed kernel.
  * ``direct_circ`` / ``fftconv_circ`` -- the circular mode (summary, "Boundary
    handling": periodic grids, no padding): y[i] = sum_j u[j] K[(i-j) mod n]
    with K stored [C, *dims], index m = offset mod n.
  * ``direct_per_sample`` / ``fftconv_per_sample`` -- input-dependent kernels
    (summary, "Input dependent kernels via registers and FiLM": the kernel is
    conditioned on the whole sample): y[b,c,i] = sum_j u[b,c,j] K[b,c][i-j],
    K [B, C, *(2n-1)]; O1 / O2 applied per batch entry with that entry's kernels.
  * ``bwd_direct_per_sample`` / ``bwd_fft_per_sample`` -- their backward: the
    shared-kernel backward per batch entry with that entry's kernels, dK kept
    per (b, c), dalpha and dbeta summed over the batch (the parameters are
    shared by every sample).
  * ``bwd_direct_circ`` / ``bwd_fft_circ`` -- the backward of the circular mode
    (offsets modulo n; dK on the n offsets).
  * ``bwd_direct`` / ``bwd_points`` / ``bwd_fft`` -- the backward (vector-Jacobian
    product, explainer section "Implementation and operation patterns", item
    "Concrete implementation pattern (PyTorch)": gradients of the input and of
    the kernel parameters): O1 written out (all, or chosen points) and O2 by
    FFTs.  Given dy = dLoss/dy::

        du[j]    = sum_i dy[i] K[i-j]
        dx[j]    = du[j] (s + alpha x s (1-s)),   s = sigmoid(alpha x + beta)
        dalpha_c = sum_{b,j} du x^2 s (1-s),   dbeta_c = sum_{b,j} du x s (1-s)
        dK_c[l]  = sum_b sum_j dy[j+l] u[j]     (l over K's offsets)

Inputs are numpy arrays: x fp32 [B,C,*dims] (bf16 data widened exactly to fp32
by the caller), alpha/beta fp32 [C], K fp32 [C,*(2*dims-1)].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc -O2 -fopenmp."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_gate.argtypes = [P, I64, ctypes.c_double, ctypes.c_double, P]
        lib.oracle_gate_vjp.argtypes = [P, P, I64, ctypes.c_double, ctypes.c_double, P, P]
        lib.oracle_generate_kernels.argtypes = [P, I, I, I, P, I, I] + [P] * 10 + [ctypes.c_double, P]
        lib.oracle_direct.argtypes = [P, P, P, P, P, I, I, I, P]
        lib.oracle_direct_points.argtypes = [P, P, P, P, I, I, I, P, I64, P, P]
        lib.oracle_kernel_spectrum.argtypes = [P, I, I, P, P, P]
        lib.oracle_fftconv_pairs.argtypes = [P, P, P, P, I, I, I, P, I64, P, P]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_direct_circ.argtypes = [P, P, P, P, P, I, I, I, P]
        lib.oracle_bwd_direct_circ.argtypes = [P, P, P, P, P, I, I, I, P, P, P, P, P]
        lib.oracle_bwd_fft_circ.argtypes = [P, P, P, P, P, I, I, I, P, I64, P, P, P, P, P]
        lib.oracle_fftconv_circ_pairs.argtypes = [P, P, P, P, I, I, I, P, I64, P, P]
        lib.oracle_bwd_direct.argtypes = [P, P, P, P, P, I, I, I, P, P, P, P, P]
        lib.oracle_bwd_direct_points.argtypes = [P, P, P, P, P, I, I, I, P, I64, P, P, I64, P, P]
        lib.oracle_bwd_fft.argtypes = [P, P, P, P, P, I, I, I, P, I64, P, P, P, P, P]
        for f in ("oracle_gate", "oracle_gate_vjp", "oracle_generate_kernels", "oracle_direct", "oracle_direct_points", "oracle_kernel_spectrum",
                  "oracle_fftconv_pairs", "oracle_num_threads", "oracle_bwd_direct", "oracle_bwd_direct_points",
                  "oracle_bwd_fft", "oracle_direct_circ", "oracle_fftconv_circ_pairs", "oracle_bwd_direct_circ",
                  "oracle_bwd_fft_circ"):
            getattr(lib, f).restype = I
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _dims_of(x: np.ndarray, d: int):
    dims = np.ascontiguousarray(np.asarray(x.shape[2:], dtype=np.int64))
    if dims.size != d:
        raise ValueError("x must be [B, C, *dims]")
    return dims


def gate(x, alpha: float, beta: float) -> np.ndarray:
    """u = phi(x) * x, phi the logistic of alpha*x + beta, in fp64."""
    x = _f32(x)
    u = np.empty(x.shape, dtype=np.float64)
    _check(_load().oracle_gate(_ptr(x), x.size, float(alpha), float(beta), _ptr(u)), "gate")
    return u


def gate_vjp(x, du, alpha: float, beta: float):
    """The gate's backward alone: for u = phi(x) x and an output gradient du
    (same shape as x), returns (dx, sum du x^2 s(1-s), sum du x s(1-s)), s the
    logistic of alpha*x + beta, in fp64 (the chain rule written out in the
    backward section of oracle.c)."""
    x = _f32(x)
    du = np.ascontiguousarray(np.asarray(du, dtype=np.float64))
    if du.shape != x.shape:
        raise ValueError("du must have the shape of x")
    dx = np.empty(x.shape, dtype=np.float64)
    sums = np.zeros(2, dtype=np.float64)
    _check(_load().oracle_gate_vjp(_ptr(x), _ptr(du), x.size, float(alpha), float(beta), _ptr(dx), _ptr(sums)),
           "gate_vjp")
    return dx, float(sums[0]), float(sums[1])


def direct(x, alpha, beta, K) -> np.ndarray:
    """O1: every output of the gated linear convolution, fp64 [B, C, *dims]."""
    x, alpha, beta, K = _f32(x), _f32(alpha), _f32(beta), _f32(K)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    y = np.empty(x.shape, dtype=np.float64)
    _check(_load().oracle_direct(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), _ptr(y), B, C, d, _ptr(dims)),
           "direct")
    return y


def direct_points(x, alpha, beta, K, points) -> np.ndarray:
    """O1 at chosen outputs; ``points`` is int [P, 2+d] rows (b, c, i_0..i_{d-1})."""
    x, alpha, beta, K = _f32(x), _f32(alpha), _f32(beta), _f32(K)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    pts = np.ascontiguousarray(np.asarray(points, dtype=np.int64).reshape(-1, 2 + d))
    out = np.empty(pts.shape[0], dtype=np.float64)
    _check(_load().oracle_direct_points(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), B, C, d, _ptr(dims),
                                        pts.shape[0], _ptr(pts), _ptr(out)), "direct_points")
    return out


def fftconv(x, alpha, beta, K, pairs=None) -> np.ndarray:
    """O2 for the listed pair indices (b*C + c); all pairs when ``pairs`` is None.

    Returns fp64 [len(pairs), *dims] (or [B, C, *dims] for all pairs).
    """
    x, alpha, beta, K = _f32(x), _f32(alpha), _f32(beta), _f32(K)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    allp = pairs is None
    pr = np.arange(B * C, dtype=np.int64) if allp else np.ascontiguousarray(np.asarray(pairs, dtype=np.int64))
    y = np.empty((pr.size,) + tuple(x.shape[2:]), dtype=np.float64)
    _check(_load().oracle_fftconv_pairs(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), B, C, d, _ptr(dims),
                                        pr.size, _ptr(pr), _ptr(y)), "fftconv")
    return y.reshape(x.shape) if allp else y


def kernel_spectrum(K, dims) -> np.ndarray:
    """Full DFT (complex128 [C, *2*dims]) of each channel's wrap-placed kernel."""
    K = _f32(K)
    d = len(dims)
    dd = np.ascontiguousarray(np.asarray(dims, dtype=np.int64))
    C = K.shape[0]
    shape = (C,) + tuple(2 * int(n) for n in dims)
    re = np.empty(shape, dtype=np.float64)
    im = np.empty(shape, dtype=np.float64)
    _check(_load().oracle_kernel_spectrum(_ptr(K), C, d, _ptr(dd), _ptr(re), _ptr(im)), "kernel_spectrum")
    return re + 1j * im


GEN_HIDDEN = 16
GEN_KEYS = ("Wreg", "breg", "q", "Wgam", "Wbet", "W1", "b1", "W2", "b2", "sigma")


def generate_kernels(x, gen) -> np.ndarray:
    """Input-dependent kernels (summary, "Methodology": registers, a
    softmax-weighted control z(x), a FiLM-modulated SIREN, a Gaussian window;
    the steps are spelled out in oracle.c): x [B, C, *dims] and the generator
    parameters ``gen`` (dict of arrays: Wreg [R, D, C], breg [R, D], q [D],
    Wgam [16, D], Wbet [16, D], W1 [16, d], b1 [16], W2 [C, 16], b2 [C],
    sigma [C], and the scalar omega0) -> K fp64 [B, C, *(2n-1)]."""
    x = _f32(x)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    arrs = {k: _f32(gen[k]) for k in GEN_KEYS}
    R, D = arrs["Wreg"].shape[:2]
    if arrs["Wreg"].shape != (R, D, C) or arrs["W1"].shape != (GEN_HIDDEN, d) or arrs["W2"].shape != (C, GEN_HIDDEN):
        raise ValueError("generator parameter shapes")
    K = np.empty((B, C) + tuple(2 * int(n) - 1 for n in dims), dtype=np.float64)
    _check(_load().oracle_generate_kernels(_ptr(x), B, C, d, _ptr(dims), R, D,
                                           *[_ptr(arrs[k]) for k in GEN_KEYS], float(gen["omega0"]), _ptr(K)),
           "generate_kernels")
    return K


def direct_per_sample(x, alpha, beta, K) -> np.ndarray:
    """O1 with one kernel per (b, c): K [B, C, *(2n-1)] -> fp64 [B, C, *dims]."""
    x, K = _f32(x), _f32(K)
    if K.shape[:2] != x.shape[:2]:
        raise ValueError("per-sample kernels are [B, C, *(2n-1)]")
    return np.concatenate([direct(x[b:b + 1], alpha, beta, K[b]) for b in range(x.shape[0])], axis=0)


def fftconv_per_sample(x, alpha, beta, K, batch=None) -> np.ndarray:
    """O2 with one kernel per (b, c), for the listed batch entries (all when None): fp64 [len, C, *dims]."""
    x, K = _f32(x), _f32(K)
    if K.shape[:2] != x.shape[:2]:
        raise ValueError("per-sample kernels are [B, C, *(2n-1)]")
    bs = range(x.shape[0]) if batch is None else batch
    return np.concatenate([fftconv(x[b:b + 1], alpha, beta, K[b]) for b in bs], axis=0)


def _bwd_per_sample(route, x, alpha, beta, K, dy, batch):
    x, K, dy = _f32(x), _f32(K), _f32(dy)
    if K.shape[:2] != x.shape[:2] or dy.shape != x.shape:
        raise ValueError("per-sample kernels are [B, C, *(2n-1)], dy is shaped like x")
    bs = range(x.shape[0]) if batch is None else batch
    parts = [route(x[b:b + 1], alpha, beta, K[b], dy[b:b + 1]) for b in bs]
    dx = np.concatenate([p[0] for p in parts], axis=0)
    da = np.sum([p[1] for p in parts], axis=0)
    db = np.sum([p[2] for p in parts], axis=0)
    dK = np.stack([p[3] for p in parts])
    return dx, da, db, dK


def bwd_direct_per_sample(x, alpha, beta, K, dy, batch=None):
    """O1 backward with one kernel per (b, c), for the listed batch entries (all
    when None): (dx [len, C, *dims], dalpha [C], dbeta [C] summed over those
    entries, dK [len, C, *(2n-1)]), fp64."""
    return _bwd_per_sample(bwd_direct, x, alpha, beta, K, dy, batch)


def bwd_fft_per_sample(x, alpha, beta, K, dy, batch=None):
    """O2 backward with one kernel per (b, c); outputs as bwd_direct_per_sample."""
    return _bwd_per_sample(bwd_fft, x, alpha, beta, K, dy, batch)


def direct_circ(x, alpha, beta, K) -> np.ndarray:
    """O1, circular mode: every output, fp64 [B, C, *dims]; K is [C, *dims] (index = offset mod n)."""
    x, alpha, beta, K = _f32(x), _f32(alpha), _f32(beta), _f32(K)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    if tuple(K.shape) != (C,) + tuple(x.shape[2:]):
        raise ValueError("the circular kernel is [C, *dims]")
    y = np.empty(x.shape, dtype=np.float64)
    _check(_load().oracle_direct_circ(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), _ptr(y), B, C, d, _ptr(dims)),
           "direct_circ")
    return y


def fftconv_circ(x, alpha, beta, K, pairs=None) -> np.ndarray:
    """O2, circular mode (FFT of size n, no padding) for the listed pairs (all when None)."""
    x, alpha, beta, K = _f32(x), _f32(alpha), _f32(beta), _f32(K)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    if tuple(K.shape) != (C,) + tuple(x.shape[2:]):
        raise ValueError("the circular kernel is [C, *dims]")
    allp = pairs is None
    pr = np.arange(B * C, dtype=np.int64) if allp else np.ascontiguousarray(np.asarray(pairs, dtype=np.int64))
    y = np.empty((pr.size,) + tuple(x.shape[2:]), dtype=np.float64)
    _check(_load().oracle_fftconv_circ_pairs(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), B, C, d, _ptr(dims),
                                             pr.size, _ptr(pr), _ptr(y)), "fftconv_circ")
    return y.reshape(x.shape) if allp else y


def bwd_direct(x, alpha, beta, K, dy):
    """O1 backward: (dx [B,C,*dims], dalpha [C], dbeta [C], dK [C,*(2*dims-1)]), fp64."""
    x, alpha, beta, K, dy = _f32(x), _f32(alpha), _f32(beta), _f32(K), _f32(dy)
    if dy.shape != x.shape:
        raise ValueError("dy must have the shape of x")
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    dx = np.empty(x.shape, dtype=np.float64)
    da = np.empty(C, dtype=np.float64)
    db = np.empty(C, dtype=np.float64)
    dK = np.empty(K.shape, dtype=np.float64)
    _check(_load().oracle_bwd_direct(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), _ptr(dy), B, C, d, _ptr(dims),
                                     _ptr(dx), _ptr(da), _ptr(db), _ptr(dK)), "bwd_direct")
    return dx, da, db, dK


def bwd_points(x, alpha, beta, K, dy, x_points=None, k_points=None):
    """O1 backward at chosen points: dx at rows (b, c, j_0..) and dK at rows (c, e_0..)
    (e the index into K's extents).  Returns (dx values, dK values), fp64."""
    x, alpha, beta, K, dy = _f32(x), _f32(alpha), _f32(beta), _f32(K), _f32(dy)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    xp = np.ascontiguousarray(np.asarray([] if x_points is None else x_points, dtype=np.int64).reshape(-1, 2 + d))
    kp = np.ascontiguousarray(np.asarray([] if k_points is None else k_points, dtype=np.int64).reshape(-1, 1 + d))
    ox = np.empty(max(xp.shape[0], 1), dtype=np.float64)
    ok = np.empty(max(kp.shape[0], 1), dtype=np.float64)
    _check(_load().oracle_bwd_direct_points(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), _ptr(dy), B, C, d,
                                            _ptr(dims), xp.shape[0], _ptr(xp), _ptr(ox), kp.shape[0], _ptr(kp),
                                            _ptr(ok)), "bwd_points")
    return ox[:xp.shape[0]], ok[:kp.shape[0]]


def bwd_fft(x, alpha, beta, K, dy, chans=None):
    """O2 backward for the listed channels (all when None), every batch entry.

    Returns (dx [B, len(chans), *dims], dalpha [len], dbeta [len], dK [len, *(2*dims-1)]), fp64.
    """
    x, alpha, beta, K, dy = _f32(x), _f32(alpha), _f32(beta), _f32(K), _f32(dy)
    if dy.shape != x.shape:
        raise ValueError("dy must have the shape of x")
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    ch = np.arange(C, dtype=np.int64) if chans is None else np.ascontiguousarray(np.asarray(chans, dtype=np.int64))
    n = ch.size
    dx = np.empty((n, B) + tuple(x.shape[2:]), dtype=np.float64)
    da = np.empty(n, dtype=np.float64)
    db = np.empty(n, dtype=np.float64)
    dK = np.empty((n,) + tuple(K.shape[1:]), dtype=np.float64)
    _check(_load().oracle_bwd_fft(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), _ptr(dy), B, C, d, _ptr(dims),
                                  n, _ptr(ch), _ptr(dx), _ptr(da), _ptr(db), _ptr(dK)), "bwd_fft")
    return np.ascontiguousarray(dx.swapaxes(0, 1)), da, db, dK


def bwd_direct_circ(x, alpha, beta, K, dy):
    """O1 backward of the circular mode: (dx, dalpha, dbeta, dK [C, *dims]), fp64."""
    x, alpha, beta, K, dy = _f32(x), _f32(alpha), _f32(beta), _f32(K), _f32(dy)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    if dy.shape != x.shape or tuple(K.shape) != (C,) + tuple(x.shape[2:]):
        raise ValueError("dy is shaped like x, the circular kernel [C, *dims]")
    dx = np.empty(x.shape, dtype=np.float64)
    da = np.empty(C, dtype=np.float64)
    db = np.empty(C, dtype=np.float64)
    dK = np.empty(K.shape, dtype=np.float64)
    _check(_load().oracle_bwd_direct_circ(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), _ptr(dy), B, C, d, _ptr(dims),
                                          _ptr(dx), _ptr(da), _ptr(db), _ptr(dK)), "bwd_direct_circ")
    return dx, da, db, dK


def bwd_fft_circ(x, alpha, beta, K, dy, chans=None):
    """O2 backward of the circular mode for the listed channels (all when None):
    (dx [B, len, *dims], dalpha [len], dbeta [len], dK [len, *dims]), fp64."""
    x, alpha, beta, K, dy = _f32(x), _f32(alpha), _f32(beta), _f32(K), _f32(dy)
    B, C = x.shape[:2]
    d = x.ndim - 2
    dims = _dims_of(x, d)
    ch = np.arange(C, dtype=np.int64) if chans is None else np.ascontiguousarray(np.asarray(chans, dtype=np.int64))
    n = ch.size
    dx = np.empty((n, B) + tuple(x.shape[2:]), dtype=np.float64)
    da = np.empty(n, dtype=np.float64)
    db = np.empty(n, dtype=np.float64)
    dK = np.empty((n,) + tuple(x.shape[2:]), dtype=np.float64)
    _check(_load().oracle_bwd_fft_circ(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(K), _ptr(dy), B, C, d, _ptr(dims),
                                       n, _ptr(ch), _ptr(dx), _ptr(da), _ptr(db), _ptr(dK)), "bwd_fft_circ")
    return np.ascontiguousarray(dx.swapaxes(0, 1)), da, db, dK


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())
