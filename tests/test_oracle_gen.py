"""Pins for the oracle's input-dependent kernel generator (gist.science
summary of the paper, "Methodology": registers prepended to the input, a
control variable z(x) as a softmax-weighted mean of the register activations,
FiLM modulation of a coordinate SIREN, and K(x) = w(c) (.) f(c; z(x)) with a
Gaussian window w).  Each pin checks a closed form or an invariance that a
plausible slip in the generator would break, computed by scalar Python math
(not by the oracle's loops); the planted-mistake test shows each pin has
teeth."""
import math

import numpy as np
import pytest

import oracle
import synth


def _x(B, C, dims, seed, shift=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, C) + tuple(dims)).astype(np.float32)
    if shift:  # per-sample offsets, so the samples' statistics differ
        x += np.arange(B, dtype=np.float32).reshape((B,) + (1,) * (len(dims) + 1)) * 0.7
    return x


def _siren(gen, c, delta, dims, gam, bet):
    """f(c; z)(delta) for one offset, by scalar math."""
    f = float(gen["b2"][c])
    for k in range(16):
        arg = float(gen["b1"][k]) + sum(float(gen["W1"][k, a]) * delta[a] / (dims[a] - 1) for a in range(len(dims)))
        f += float(gen["W2"][c, k]) * (gam[k] * math.sin(gen["omega0"] * arg) + bet[k])
    return f


def _window(gen, c, delta):
    return math.exp(-sum(v * v for v in delta) / (2.0 * float(gen["sigma"][c]) ** 2))


def _offsets(dims, count, seed):
    rng = np.random.default_rng(seed)
    return [tuple(int(rng.integers(-(n - 1), n)) for n in dims) for _ in range(count)] + \
           [tuple(0 for _ in dims), tuple(n - 1 for n in dims), tuple(-(n - 1) for n in dims)]


def _at(K, b, c, delta, dims):
    return K[(b, c) + tuple(v + n - 1 for v, n in zip(delta, dims))]


@pytest.mark.parametrize("dims", [(9,), (5, 8), (4, 3, 6)])
def test_film_identity_is_the_plain_siren_times_window(dims):
    """Wgam = Wbet = 0: gamma = 1, beta = 0 whatever z, so K is the same for
    every sample and equals w(delta) (b2 + sum_k W2 sin(omega0 (W1 chat + b1)))."""
    C, B = 3, 2
    gen = synth.draw_generator(dims, C, seed=1)
    gen["Wgam"] = np.zeros_like(gen["Wgam"])
    gen["Wbet"] = np.zeros_like(gen["Wbet"])
    K = oracle.generate_kernels(_x(B, C, dims, 2), gen)
    assert np.array_equal(K[0], K[1])
    for c in range(C):
        for delta in _offsets(dims, 12, c):
            want = _window(gen, c, delta) * _siren(gen, c, delta, dims, [1.0] * 16, [0.0] * 16)
            assert abs(_at(K, 0, c, delta, dims) - want) <= 1e-12 * max(1.0, abs(want))


def test_constant_registers_give_z_equal_to_the_register():
    """Wreg = 0 and identical register biases: every register holds
    a = tanh(breg), the softmax weights are uniform whatever q, so z = a; with
    a one-hot readout W2[c] = e_k and b2 = 0, K = w (gamma_k h_k + beta_k) with
    gamma_k = 1 + Wgam[k] . a and beta_k = Wbet[k] . a (closed form)."""
    dims, C, B, R, D = (6, 7), 2, 3, 5, 4
    gen = synth.draw_generator(dims, C, seed=3, R=R, D=D)
    gen["Wreg"] = np.zeros_like(gen["Wreg"])
    row = gen["breg"][0].copy()
    gen["breg"] = np.tile(row, (R, 1))
    gen["b2"] = np.zeros_like(gen["b2"])
    gen["W2"] = np.zeros_like(gen["W2"])
    ks = [5, 11]
    for c, k in enumerate(ks):
        gen["W2"][c, k] = 1.0
    K = oracle.generate_kernels(_x(B, C, dims, 4), gen)
    a = np.tanh(row.astype(np.float64))
    for c, k in enumerate(ks):
        gam = 1.0 + float(np.dot(gen["Wgam"][k].astype(np.float64), a))
        bet = float(np.dot(gen["Wbet"][k].astype(np.float64), a))
        for delta in _offsets(dims, 10, 7 + c):
            arg = float(gen["b1"][k]) + sum(float(gen["W1"][k, ax]) * delta[ax] / (dims[ax] - 1) for ax in range(2))
            want = _window(gen, c, delta) * (gam * math.sin(gen["omega0"] * arg) + bet)
            for b in range(B):
                assert abs(_at(K, b, c, delta, dims) - want) <= 1e-12 * max(1.0, abs(want))


def test_window_alone():
    """W2 = 0, b2 = 1: K = exp(-|delta|^2 / (2 sigma_c^2)) exactly."""
    dims, C = (5, 4, 3), 2
    gen = synth.draw_generator(dims, C, seed=5)
    gen["W2"] = np.zeros_like(gen["W2"])
    gen["b2"] = np.ones_like(gen["b2"])
    K = oracle.generate_kernels(_x(1, C, dims, 6), gen)
    for c in range(C):
        for delta in _offsets(dims, 10, c):
            assert abs(_at(K, 0, c, delta, dims) - _window(gen, c, delta)) <= 1e-15


def test_register_order_does_not_matter():
    """z is a softmax-weighted mean over the registers: permuting them (Wreg,
    breg together) leaves every kernel unchanged; and the samples' kernels
    differ once their statistics do."""
    dims, C, B = (8, 8), 3, 2
    gen = synth.draw_generator(dims, C, seed=9)
    x = _x(B, C, dims, 10)
    K = oracle.generate_kernels(x, gen)
    perm = [2, 0, 3, 1]
    gp = dict(gen, Wreg=gen["Wreg"][perm], breg=gen["breg"][perm])
    assert np.max(np.abs(oracle.generate_kernels(x, gp) - K)) <= 1e-12 * np.max(np.abs(K))
    assert np.max(np.abs(K[0] - K[1])) > 1e-3 * np.max(np.abs(K))


def test_control_is_the_softmax_weighted_register_mean():
    """Two registers with the score difference q . (a_0 - a_1) = t: z =
    sigmoid(t) a_0 + sigmoid(-t) a_1 (softmax of two scores); checked through
    gamma_k with a one-hot readout, D = 1 so every quantity is a scalar."""
    dims, C, R, D = (4, 5), 1, 2, 1
    gen = synth.draw_generator(dims, C, seed=11, R=R, D=D)
    gen["Wreg"] = np.zeros_like(gen["Wreg"])
    gen["breg"] = np.array([[0.3], [-0.8]], np.float32)
    gen["q"] = np.array([1.7], np.float32)
    gen["Wbet"] = np.zeros_like(gen["Wbet"])
    gen["W2"] = np.zeros_like(gen["W2"])
    gen["W2"][0, 3] = 1.0
    gen["b2"] = np.zeros_like(gen["b2"])
    K = oracle.generate_kernels(_x(1, C, dims, 12), gen)
    f32 = lambda v: float(np.float32(v))  # the oracle reads fp32 parameters
    a0, a1 = math.tanh(f32(0.3)), math.tanh(f32(-0.8))
    t = f32(1.7) * (a0 - a1)
    z = a0 / (1 + math.exp(-t)) + a1 / (1 + math.exp(t))
    gam = 1.0 + float(gen["Wgam"][3, 0]) * z
    for delta in _offsets(dims, 8, 13):
        arg = float(gen["b1"][3]) + sum(float(gen["W1"][3, ax]) * delta[ax] / (dims[ax] - 1) for ax in range(2))
        want = _window(gen, 0, delta) * gam * math.sin(gen["omega0"] * arg)
        assert abs(_at(K, 0, 0, delta, dims) - want) <= 1e-12 * max(1.0, abs(want))


def _pins_hold(generate):
    """Run the closed-form pins above against a generator function."""
    try:
        dims, C = (5, 8), 2
        gen = synth.draw_generator(dims, C, seed=1)
        g0 = dict(gen, Wgam=np.zeros_like(gen["Wgam"]), Wbet=np.zeros_like(gen["Wbet"]))
        K = generate(_x(2, C, dims, 2), g0)
        for c in range(C):
            for delta in _offsets(dims, 6, c):
                want = _window(g0, c, delta) * _siren(g0, c, delta, dims, [1.0] * 16, [0.0] * 16)
                if abs(_at(K, 0, c, delta, dims) - want) > 1e-9 * max(1.0, abs(want)):
                    return False
        gw = dict(gen, W2=np.zeros_like(gen["W2"]), b2=np.ones_like(gen["b2"]))
        Kw = generate(_x(1, C, dims, 6), gw)
        for delta in _offsets(dims, 6, 3):
            if abs(_at(Kw, 0, 0, delta, dims) - _window(gw, 0, delta)) > 1e-12:
                return False
        R = gen["Wreg"].shape[0]
        gz = dict(gen, Wreg=np.zeros_like(gen["Wreg"]), breg=np.tile(gen["breg"][0], (R, 1)),
                  b2=np.zeros_like(gen["b2"]), W2=np.eye(16, dtype=np.float32)[[4, 9]])
        Kz = generate(_x(2, C, dims, 4), gz)
        a = np.tanh(gen["breg"][0].astype(np.float64))
        for c, k in enumerate((4, 9)):
            gam = 1.0 + float(np.dot(gen["Wgam"][k].astype(np.float64), a))
            bet = float(np.dot(gen["Wbet"][k].astype(np.float64), a))
            for delta in _offsets(dims, 6, 8):
                arg = float(gen["b1"][k]) + sum(float(gen["W1"][k, ax]) * delta[ax] / (dims[ax] - 1) for ax in range(2))
                want = _window(gz, c, delta) * (gam * math.sin(gen["omega0"] * arg) + bet)
                if abs(_at(Kz, 1, c, delta, dims) - want) > 1e-9 * max(1.0, abs(want)):
                    return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("mutant", ["window_without_two", "film_shift_dropped", "z_not_softmax", "chat_unscaled"])
def test_pins_reject_mutants(mutant):
    """Mistakes planted in the oracle's inputs or outputs: a window
    exp(-|d|^2 / sigma^2), a FiLM with the shift beta dropped, a control z
    taken as the plain mean (q = 0 would hide nothing here: the register
    activations are shifted), and coordinates not divided by (n - 1)."""
    assert _pins_hold(oracle.generate_kernels)

    def gen_mut(x, gen):
        g = dict(gen)
        if mutant == "window_without_two":
            g["sigma"] = gen["sigma"] / np.float32(math.sqrt(2.0))
        elif mutant == "film_shift_dropped":
            g["Wbet"] = np.zeros_like(gen["Wbet"])
        elif mutant == "z_not_softmax":
            g["breg"] = gen["breg"] + np.float32(0.25)
        elif mutant == "chat_unscaled":
            dims = x.shape[2:]
            g["W1"] = gen["W1"] * np.asarray([n - 1 for n in dims], np.float32)
        return oracle.generate_kernels(x, g)

    assert not _pins_hold(gen_mut)
