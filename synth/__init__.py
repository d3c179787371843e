"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws the inputs of record and nothing else: it holds none of the
convolution's arithmetic (no gate, no transform, no product).  Both the GPU
library and the CPU oracle receive the arrays it returns.

Workload shapes stand in for the pages' examples: the 256x256 image whose cost
the explainer ("Native multi-dimensional subquadratic operators via
input-dependent long convolutions", section "HyenaND: native-space implicit
global kernel", complexity analysis) works out, and the 512^3 CT volume of its
problem statement section.  The public datasets of the summary's results section
are not used.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per config, fixed order):
  alpha[C], beta[C] ~ U(-1, 1)         per-channel gate parameters
  lam[C]            ~ U(0.01, 0.2)     per-channel window decay (voxel units)
  W1[16, d]         ~ U(-1, 1)         sine layer weights, shared by channels
  b1[16]            ~ U(-pi, pi)       sine layer bias
  W2[C, 16]         ~ U(-1/4, 1/4)     per-channel read-out, bias 0
  x[B, C, *dims]    ~ N(0, 1) fp32, rounded to bf16 (nearest even) for bf16 I/O

The kernel of channel c on integer offsets delta in [-(n-1), n-1]^d is

  K_c(delta) = (sum_k W2[c,k] sin(w0 (W1[k] . chat + b1[k]))) * exp(-lam_c ||delta||_2),
  chat_a = delta_a / (n_a - 1),  w0 = 10,

a two-layer sine MLP on continuous coordinates times a decaying window (the
summary's "Methodology" describes a SIREN kernel on continuous coordinates times
a window; the explainer's "Implementation and operation patterns" lists MLP
kernels).  It is evaluated in fp64 and rounded once to fp32; that fp32 array is
the input of record for both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HIDDEN = 16
OMEGA0 = 10.0


@dataclass(frozen=True)
class Workload:
    name: str
    dims: tuple
    B: int
    C: int
    dtype: str  # "f32" or "bf16"
    seed: int

    @property
    def d(self) -> int:
        return len(self.dims)

    @property
    def voxels(self) -> int:
        return int(np.prod(self.dims))


# The five seeded workloads: a 32^2 correctness case, the 256^2 image, a 1024^2
# multi-pass case in bf16, the 128^3 volume and the 512^3 CT volume in bf16.
WORKLOADS = [
    Workload("2d_32x32_b1_c4_f32", (32, 32), 1, 4, "f32", 1000),
    Workload("2d_256x256_b8_c64_f32", (256, 256), 8, 64, "f32", 1001),
    Workload("2d_1024x1024_b2_c128_bf16", (1024, 1024), 2, 128, "bf16", 1002),
    Workload("3d_128x128x128_b1_c32_f32", (128, 128, 128), 1, 32, "f32", 1003),
    Workload("3d_512x512x512_b1_c4_bf16", (512, 512, 512), 1, 4, "bf16", 1004),
    # long 1-D sequence (the summary's genomics context, "Results": throughput up to 10M tokens)
    Workload("1d_2097152_b1_c8_bf16", (2097152,), 1, 8, "bf16", 1005),
    Workload("1d_8388608_b1_c4_bf16", (8388608,), 1, 4, "bf16", 1006),
    # the explainer's volumetric examples ("Quantified performance impact": a
    # 512x512x64 tensor of 16M voxels in fp32; "Empirical validation": a
    # 1024x1024x256 climate grid); the pages give no channel count
    Workload("3d_512x512x64_b1_c16_f32", (512, 512, 64), 1, 16, "f32", 1007),
    Workload("3d_1024x1024x256_b1_c2_f32", (1024, 1024, 256), 1, 2, "f32", 1008),
    # smaller images with the 256^2 image's batch and channels: 128^2 (three
    # passes) and 64^2 (the largest grid of the on-chip 2-D forward)
    Workload("2d_128x128_b8_c64_f32", (128, 128), 8, 64, "f32", 1009),
    Workload("2d_64x64_b8_c64_f32", (64, 64), 8, 64, "f32", 1010),
    # 2^24 tokens: the summary's 10M-token genomics context, zero-extended to a
    # power of two (outputs below 10M are those of the 10M-token problem)
    Workload("1d_16777216_b1_c2_bf16", (16777216,), 1, 2, "bf16", 1011),
]


@dataclass
class Params:
    alpha: np.ndarray
    beta: np.ndarray
    lam: np.ndarray
    W1: np.ndarray
    b1: np.ndarray
    W2: np.ndarray
    rng: np.random.Generator = field(repr=False)


def draw_params(dims, C: int, seed: int) -> Params:
    """Draw the per-channel parameters in the fixed order; the generator is
    returned positioned for the draw of x."""
    d = len(dims)
    rng = np.random.Generator(np.random.PCG64(seed))
    alpha = rng.uniform(-1.0, 1.0, C).astype(np.float32)
    beta = rng.uniform(-1.0, 1.0, C).astype(np.float32)
    lam = rng.uniform(0.01, 0.2, C)
    W1 = rng.uniform(-1.0, 1.0, (HIDDEN, d))
    b1 = rng.uniform(-math.pi, math.pi, HIDDEN)
    W2 = rng.uniform(-0.25, 0.25, (C, HIDDEN))
    return Params(alpha, beta, lam, W1, b1, W2, rng)


def draw_x(rng: np.random.Generator, B: int, C: int, dims, dtype: str):
    """x ~ N(0,1) fp32 [B, C, *dims]; for bf16 I/O returns the bf16-rounded
    values as a torch bfloat16 tensor (round to nearest even)."""
    import torch

    x = rng.standard_normal((B, C) + tuple(dims), dtype=np.float32)
    t = torch.from_numpy(x)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


def kernel_channels(dims, p: Params, channels=None, device="cpu", out=None):
    """Materialise K_c for the listed channels as fp32 [len(channels), *(2n-1)].

    Evaluated slab by slab along the first axis in fp64 on ``device`` (a torch
    device string); ``out`` may be a preallocated fp32 torch tensor.
    """
    import torch

    d = len(dims)
    chans = list(range(p.W2.shape[0])) if channels is None else list(channels)
    ext = [2 * n - 1 for n in dims]
    dev = torch.device(device)
    f64 = torch.float64
    if out is None:
        out = torch.empty([len(chans)] + ext, dtype=torch.float32, device=dev)
    W1 = torch.tensor(p.W1, dtype=f64, device=dev)
    b1 = torch.tensor(p.b1, dtype=f64, device=dev)
    W2 = torch.tensor(p.W2[chans], dtype=f64, device=dev)
    lam = torch.tensor(p.lam[chans], dtype=f64, device=dev)
    offs = [torch.arange(-(n - 1), n, dtype=f64, device=dev) for n in dims]
    chat = [o / (n - 1) if n > 1 else torch.zeros_like(o) for o, n in zip(offs, dims)]
    if d == 1:
        # One axis: evaluate the offsets in blocks (a slab per offset would be
        # millions of tiny steps for long signals).
        step = 1 << 18
        for s0 in range(0, ext[0], step):
            o, ch = offs[0][s0:s0 + step], chat[0][s0:s0 + step]
            h = torch.sin(OMEGA0 * (b1.reshape(HIDDEN, 1) + W1[:, 0].reshape(HIDDEN, 1) * ch.reshape(1, -1)))
            mlp = torch.tensordot(W2, h, dims=([1], [0]))             # [C', block]
            win = torch.exp(-lam.reshape(-1, 1) * torch.sqrt(o ** 2).reshape(1, -1))
            out[:, s0:s0 + step] = (mlp * win).to(torch.float32)
        return out
    # Contribution of the trailing axes to the sine argument and to ||delta||^2.
    rest_arg = torch.zeros([HIDDEN] + ext[1:], dtype=f64, device=dev)
    rest_r2 = torch.zeros(ext[1:], dtype=f64, device=dev)
    for a in range(1, d):
        shape = [1] * (d - 1)
        shape[a - 1] = ext[a]
        rest_arg = rest_arg + W1[:, a].reshape([HIDDEN] + [1] * (d - 1)) * chat[a].reshape([1] + shape)
        rest_r2 = rest_r2 + (offs[a] ** 2).reshape(shape)
    rest_arg = rest_arg + b1.reshape([HIDDEN] + [1] * (d - 1))
    for i0 in range(ext[0]):
        arg = rest_arg + (W1[:, 0] * chat[0][i0]).reshape([HIDDEN] + [1] * (d - 1))
        h = torch.sin(OMEGA0 * arg)                                   # [16, *rest]
        mlp = torch.tensordot(W2, h, dims=([1], [0]))                 # [C', *rest]
        r = torch.sqrt(rest_r2 + offs[0][i0] ** 2)
        win = torch.exp(-lam.reshape([-1] + [1] * (d - 1)) * r.unsqueeze(0))
        out[:, i0] = (mlp * win).to(torch.float32)
    return out


def make(wl_or_dims, B=None, C=None, dtype="f32", seed=0, device="cpu", with_kernel=True):
    """All inputs of one workload: dict with x (torch, fp32 or bf16), alpha,
    beta (numpy fp32 [C]), K (torch fp32 [C, *(2n-1)] or None) and params."""
    if isinstance(wl_or_dims, Workload):
        wl = wl_or_dims
        dims, B, C, dtype, seed = wl.dims, wl.B, wl.C, wl.dtype, wl.seed
    else:
        dims = tuple(int(v) for v in wl_or_dims)
    p = draw_params(dims, C, seed)
    x = draw_x(p.rng, B, C, dims, dtype)
    K = kernel_channels(dims, p, device=device) if with_kernel else None
    return {"x": x, "alpha": p.alpha, "beta": p.beta, "K": K, "params": p, "dims": tuple(dims),
            "B": B, "C": C, "dtype": dtype}


def sample_points(dims, B: int, C: int, pairs, per_pair: int, seed: int, edges: bool = False) -> np.ndarray:
    """Output coordinates to check one by one: for each listed pair (b, c) the
    2^d corners, the centre, with ``edges`` the midpoint of every edge of the
    grid box (and, in 3-D, the centre of every face), and ``per_pair`` seeded
    random voxels.  Returns int64 [P, 2+d] rows (b, c, i_0..i_{d-1})."""
    rng = np.random.Generator(np.random.PCG64(seed))
    d = len(dims)
    rows = []
    # Per axis: 0 = low end, 1 = high end, 2 = middle.  An edge midpoint has
    # exactly one axis in the middle, a face centre exactly two (d = 3).
    ends = [(0, n - 1, n // 2) for n in dims]
    for (b, c) in pairs:
        for corner in range(1 << d):
            rows.append([b, c] + [(dims[a] - 1) if (corner >> a) & 1 else 0 for a in range(d)])
        rows.append([b, c] + [n // 2 for n in dims])
        if edges:
            for code in range(3 ** d):
                sel = [(code // 3 ** a) % 3 for a in range(d)]
                mids = sum(1 for v in sel if v == 2)
                if 1 <= mids <= max(1, d - 1):
                    rows.append([b, c] + [ends[a][sel[a]] for a in range(d)])
        for _ in range(per_pair):
            rows.append([b, c] + [int(rng.integers(0, n)) for n in dims])
    return np.asarray(rows, dtype=np.int64)


def draw_generator(dims, C: int, seed: int, R: int = 4, D: int = 8) -> dict:
    """Seeded parameters of the input-dependent kernel generator (registers,
    softmax control, FiLM, SIREN, Gaussian window; the generator itself is the
    library's / the oracle's, not this module's).  One
    ``numpy.random.Generator(PCG64([seed, 4]))``, fixed order:
      Wreg [R, D, C] ~ U(-1, 1) * 4 / sqrt(C), breg [R, D] ~ U(-1, 1),
      q [D] ~ U(-2, 2), Wgam [16, D], Wbet [16, D] ~ U(-1/2, 1/2),
      W1 [16, d] ~ U(-1, 1), b1 [16] ~ U(-pi, pi), W2 [C, 16] ~ U(-1/4, 1/4),
      b2 [C] ~ U(-1/10, 1/10), sigma [C] ~ U(0.1, 0.4) * max(dims) (voxels),
      omega0 = 10 (the static kernels' SIREN frequency).
    All fp32 except omega0."""
    d = len(dims)
    rng = np.random.Generator(np.random.PCG64([seed, 4]))
    f = np.float32
    g = {
        "Wreg": (rng.uniform(-1, 1, (R, D, C)) * 4.0 / math.sqrt(C)).astype(f),
        "breg": rng.uniform(-1, 1, (R, D)).astype(f),
        "q": rng.uniform(-2, 2, D).astype(f),
        "Wgam": rng.uniform(-0.5, 0.5, (HIDDEN, D)).astype(f),
        "Wbet": rng.uniform(-0.5, 0.5, (HIDDEN, D)).astype(f),
        "W1": rng.uniform(-1, 1, (HIDDEN, d)).astype(f),
        "b1": rng.uniform(-math.pi, math.pi, HIDDEN).astype(f),
        "W2": rng.uniform(-0.25, 0.25, (C, HIDDEN)).astype(f),
        "b2": rng.uniform(-0.1, 0.1, C).astype(f),
        "sigma": (rng.uniform(0.1, 0.4, C) * max(dims)).astype(f),
        "omega0": OMEGA0,
    }
    return g


def draw_dy(dims, B: int, C: int, dtype: str, seed: int):
    """Output gradient of the backward: dy ~ N(0,1) fp32 [B, C, *dims] from its
    own stream, PCG64 seeded with [seed, 1] (x's stream is untouched); bf16 I/O
    rounds to bf16 as draw_x does."""
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    return draw_x(rng, B, C, dims, dtype)


def sample_kernel_points(dims, chans, per_chan: int, seed: int) -> np.ndarray:
    """Kernel-gradient coordinates to check one by one: for each listed channel
    the 2^d corner offsets +-(n-1), offset 0, and ``per_chan`` seeded random
    offsets.  Returns int64 [P, 1+d] rows (c, e_0..e_{d-1}), e the index into
    K's extents 2n-1 (offset e - (n-1))."""
    rng = np.random.Generator(np.random.PCG64([seed, 2]))
    d = len(dims)
    rows = []
    for c in chans:
        for corner in range(1 << d):
            rows.append([c] + [(2 * dims[a] - 2) if (corner >> a) & 1 else 0 for a in range(d)])
        rows.append([c] + [n - 1 for n in dims])
        for _ in range(per_chan):
            rows.append([c] + [int(rng.integers(0, 2 * n - 1)) for n in dims])
    return np.asarray(rows, dtype=np.int64)


def circular_kernel(dims, p: Params, device="cpu"):
    """Circular-mode kernel [C, *dims] fp32: the same generator evaluated on the
    periodic grid's minimal-image offsets (index m holds offset m for
    m <= n/2 and m - n above), i.e. a gather from the non-circular kernel of
    offsets -(n-1)..(n-1)."""
    import torch

    full = kernel_channels(dims, p, device=device)
    idx = [torch.tensor([(m if m <= n // 2 else m - n) + n - 1 for m in range(n)], device=full.device)
           for n in dims]
    out = full
    for a, ix in enumerate(idx):
        out = out.index_select(a + 1, ix)
    return out.contiguous()
