"""The seeded input generators: shapes, determinism and the bf16 rounding rule."""
import numpy as np
import torch

import synth


def test_shapes_and_determinism():
    a = synth.make((8, 16), B=2, C=3, dtype="f32", seed=7)
    b = synth.make((8, 16), B=2, C=3, dtype="f32", seed=7)
    assert a["x"].shape == (2, 3, 8, 16) and a["x"].dtype == torch.float32
    assert a["K"].shape == (3, 15, 31) and a["K"].dtype == torch.float32
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["K"], b["K"])
    assert np.array_equal(a["alpha"], b["alpha"])
    assert np.all(np.abs(a["alpha"]) <= 1) and np.all(np.abs(a["beta"]) <= 1)
    c = synth.make((8, 16), B=2, C=3, dtype="f32", seed=8)
    assert not torch.equal(a["x"], c["x"])


def test_kernel_window_and_centre():
    # Window exp(-lam ||delta||) with lam >= 0.01 bounds |K| by the MLP read-out
    # (16 units, |W2| <= 1/4), and the kernel decays away from the centre.
    w = synth.make((32, 32), B=1, C=4, seed=3)
    K = w["K"].numpy()
    assert np.all(np.abs(K) <= 4.0 + 1e-6)
    assert np.abs(K[:, 31, 31]).max() > 0
    p = w["params"]
    far = np.abs(K[:, 0, 0]) / np.exp(-p.lam * np.sqrt(2) * 31)
    assert np.all(far <= 4.0 + 1e-3)


def test_bf16_inputs_are_rounded_to_nearest_even():
    w = synth.make((16, 16), B=1, C=2, dtype="bf16", seed=4, with_kernel=False)
    assert w["x"].dtype == torch.bfloat16
    rng = np.random.Generator(np.random.PCG64(4))
    p = synth.draw_params((16, 16), 2, 4)
    x32 = p.rng.standard_normal((1, 2, 16, 16), dtype=np.float32)
    assert torch.equal(w["x"], torch.from_numpy(x32).to(torch.bfloat16))
    del rng


def test_kernel_slices_match_full():
    p = synth.draw_params((8, 8, 8), 3, 5)
    full = synth.kernel_channels((8, 8, 8), p)
    one = synth.kernel_channels((8, 8, 8), p, channels=[2])
    assert torch.equal(full[2:3], one)


def test_sample_points_cover_corners():
    pts = synth.sample_points((4, 8), 1, 2, [(0, 1)], per_pair=3, seed=1)
    assert pts.shape == (4 + 1 + 3, 4)
    assert [0, 1, 3, 7] in pts.tolist() and [0, 1, 0, 0] in pts.tolist()
