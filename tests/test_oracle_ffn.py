"""Pins of the blockwise-feedforward oracle (no GPU).

Against torch.nn.functional.linear and relu in float64 on the CPU (library
routines that reduce to the textbook formula), the invariance of the result
under the chunk size (the chunking only bounds memory), closed forms (W1 = 0
gives one constant row; all pre-activations negative gives b2), and planted
mistakes that must each fail a pin.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.feedforward as of


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _params(H, Fh, seed):
    return (_rand((H, Fh), seed, H ** -0.5), _rand((Fh,), seed + 1),
            _rand((Fh, H), seed + 2, Fh ** -0.5), _rand((H,), seed + 3))


def pin_ffn_torch():
    B, L, H, Fh = 2, 12, 16, 40
    x = _rand((B, L, H), 1)
    w1, b1, w2, b2 = _params(H, Fh, 10)
    t = lambda a: torch.from_numpy(a)
    ref = F.linear(F.relu(F.linear(t(x), t(w1).T.contiguous(), t(b1))), t(w2).T.contiguous(), t(b2))
    got = of.blockwise_ffn(x, w1, b1, w2, b2, 4)
    assert np.allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def pin_chunk_invariance():
    B, L, H, Fh = 2, 24, 8, 20
    x = _rand((B, L, H), 2)
    p = _params(H, Fh, 20)
    full = of.ffn(x, *p)
    for c in (1, 2, 3, 4, 6, 8, 12, 24):
        assert np.allclose(of.blockwise_ffn(x, *p, c), full, rtol=0, atol=1e-12), c


def pin_zero_w1_constant_rows():
    B, L, H, Fh = 1, 6, 8, 12
    x = _rand((B, L, H), 3)
    _, b1, w2, b2 = _params(H, Fh, 30)
    got = of.blockwise_ffn(x, np.zeros((H, Fh)), b1, w2, b2, 3)
    row = np.maximum(b1, 0.0) @ w2 + b2
    assert np.allclose(got, np.broadcast_to(row, got.shape), rtol=0, atol=1e-12)


def pin_negative_preactivation_gives_b2():
    B, L, H, Fh = 1, 4, 8, 12
    x = np.abs(_rand((B, L, H), 4))
    w1 = -np.abs(_rand((H, Fh), 40))
    b1 = -np.ones(Fh)
    _, _, w2, b2 = _params(H, Fh, 41)
    got = of.blockwise_ffn(x, w1, b1, w2, b2, 2)
    assert np.allclose(got, np.broadcast_to(b2, got.shape), rtol=0, atol=1e-12)


def pin_positive_part_only():
    """With all pre-activations positive the relu is the identity and the
    map is affine: FFN(x) = x W1 W2 + b1 W2 + b2."""
    B, L, H, Fh = 1, 5, 6, 9
    x = np.abs(_rand((B, L, H), 5))
    w1 = np.abs(_rand((H, Fh), 50))
    b1 = np.abs(_rand((Fh,), 51))
    _, _, w2, b2 = _params(H, Fh, 52)
    got = of.blockwise_ffn(x, w1, b1, w2, b2, 5)
    assert np.allclose(got, x @ (w1 @ w2) + b1 @ w2 + b2, rtol=0, atol=1e-12)


FFN_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", FFN_PINS, ids=[p.__name__ for p in FFN_PINS])
def test_pin_ffn(pin):
    pin()


def test_chunk_must_divide():
    x = np.zeros((1, 10, 4))
    p = _params(4, 6, 0)
    with pytest.raises(ValueError):
        of.blockwise_ffn(x, *p, 3)


def _mut_no_relu(mp):
    mp.setattr(of, "_relu", lambda z: z)


def _mut_relu_before_bias(mp):
    def bad(x, w1, b1, w2, b2):
        x, w1, b1, w2, b2 = (of._as_f64(t) for t in (x, w1, b1, w2, b2))
        return (np.maximum(x @ w1, 0.0) + b1) @ w2 + b2
    mp.setattr(of, "ffn", bad)


def _mut_no_b2(mp):
    orig = of.ffn
    mp.setattr(of, "ffn", lambda x, w1, b1, w2, b2: orig(x, w1, b1, w2, b2 * 0))


def _mut_chunks_reversed(mp):
    orig = of.blockwise_ffn

    def bad(x, w1, b1, w2, b2, c):
        x = of._as_f64(x)
        B, L, H = x.shape
        xc = x.reshape(B, L // c, c, H)
        out = np.stack([of.ffn(xc[:, i], w1, b1, w2, b2) for i in range(L // c)][::-1], axis=1)
        return out.reshape(B, L, H)
    mp.setattr(of, "blockwise_ffn", bad)


def _mut_leaky(mp):
    mp.setattr(of, "_relu", lambda z: np.where(z > 0, z, 0.01 * z))


FFN_MUTATIONS = [_mut_no_relu, _mut_relu_before_bias, _mut_no_b2, _mut_chunks_reversed, _mut_leaky]


@pytest.mark.parametrize("mutation", FFN_MUTATIONS, ids=[m.__name__ for m in FFN_MUTATIONS])
def test_planted_mistakes_ffn(mutation, monkeypatch):
    mutation(monkeypatch)
    failed = []
    for pin in FFN_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutation.__name__}"
