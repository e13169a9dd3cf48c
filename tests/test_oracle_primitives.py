"""Pins of the oracle's primitives against library routines and closed forms.

Every check compares the oracle with something other than itself: a torch
routine in float64 (rms_norm, silu, scaled_dot_product_attention), a complex-
number form of the rotation, or a value worked out by hand.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ref

RNG = np.random.default_rng(1234)


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# ---------------------------------------------------------------- RMSNorm

def test_rms_norm_matches_torch():
    x = RNG.standard_normal((5, 37))
    g = RNG.standard_normal(37)
    got = ref.rms_norm(x, g, 1e-6)
    want = F.rms_norm(t64(x), (37,), t64(g), 1e-6).numpy()
    assert np.max(np.abs(got - want)) < 1e-12


def test_rms_norm_hand_value_and_invariants():
    # x = (3, 4): mean square 12.5, so y = x / sqrt(12.5 + eps) * g
    y = ref.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    x = RNG.standard_normal((3, 64))
    g = np.ones(64)
    # scale invariance (eps -> 0)
    assert np.allclose(ref.rms_norm(7.5 * x, g, 0.0), ref.rms_norm(x, g, 0.0), atol=1e-13)
    # mean(y^2) = mean(x^2) / (mean(x^2) + eps)
    eps = 0.3
    ms = np.mean(x * x, axis=1)
    y = ref.rms_norm(x, g, eps)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), atol=1e-13)


# ---------------------------------------------------------------- SiLU

def test_silu_matches_torch_and_limits():
    z = np.concatenate([RNG.standard_normal(100) * 5, [0.0, -800.0, 800.0]])
    got = ref.silu(z)
    want = F.silu(t64(z)).numpy()
    assert np.max(np.abs(got - want)) < 1e-12
    assert got[-3] == 0.0 and got[-2] == 0.0 * -1 and got[-1] == 800.0


# ---------------------------------------------------------------- RoPE

def _rope_complex(x, pos, theta):
    """Rotation as complex multiplication: (x_i + i x_{i+D/2}) * exp(i p w_i)."""
    D = x.shape[-1]
    half = D // 2
    w = np.array([theta ** (-(2.0 * i) / D) for i in range(half)])
    z = x[..., :half] + 1j * x[..., half:]
    z = z * np.exp(1j * np.asarray(pos, float)[:, None, None] * w[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("D", [2, 8, 64, 128])
def test_rope_complex_form(D):
    x = RNG.standard_normal((6, 3, D))
    pos = np.array([0, 1, 5, 100, 4097, 32767])
    assert np.max(np.abs(ref.rope(x, pos, 1e6) - _rope_complex(x, pos, 1e6))) < 1e-11


def test_rope_hand_values():
    # D = 2: frequency index 0 has angle = position; rotate (1, 0) by 1 rad.
    y = ref.rope(np.array([[[1.0, 0.0]]]), [1], 1e6)
    assert np.allclose(y[0, 0], [math.cos(1.0), math.sin(1.0)], atol=1e-15)
    # D = 4, theta = 100: second pair turns by p * 100^(-1/2) = p / 10.
    x = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    y = ref.rope(x, [5], 100.0)
    assert np.allclose(y[0, 0], [0.0, math.cos(0.5), 0.0, math.sin(0.5)], atol=1e-15)


def test_rope_group_and_relative_position():
    D = 64
    x = RNG.standard_normal((1, 2, D))
    assert np.allclose(ref.rope(x, [0], 1e6), x, atol=0)
    a, b = 37, 1234
    assert np.allclose(ref.rope(ref.rope(x, [a], 1e6), [b], 1e6), ref.rope(x, [a + b], 1e6), atol=1e-11)
    assert np.allclose(np.linalg.norm(ref.rope(x, [999], 1e6), axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    q, k = RNG.standard_normal((1, 1, D)), RNG.standard_normal((1, 1, D))
    dots = []
    for shift in (0, 17, 5000):
        qm = ref.rope(q, [40 + shift], 1e6)
        kn = ref.rope(k, [3 + shift], 1e6)
        dots.append(float(np.sum(qm * kn)))
    assert np.allclose(dots, dots[0], atol=1e-11)


# ---------------------------------------------------------------- attention

def _sdpa(q, k, v, mask=None):
    # torch layout [batch, heads, seq, D]; enable_gqa maps query head h to
    # kv head h // (Hq/Hkv).
    qt = t64(q).permute(1, 0, 2)[None]
    kt = t64(k).permute(1, 0, 2)[None]
    vt = t64(v).permute(1, 0, 2)[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv,D,nq,nk", [(4, 4, 16, 8, 8), (8, 2, 32, 16, 53), (16, 2, 64, 12, 200)])
def test_attention_matches_sdpa(Hq, Hkv, D, nq, nk):
    q = RNG.standard_normal((nq, Hq, D))
    k = RNG.standard_normal((nk, Hkv, D))
    v = RNG.standard_normal((nk, Hkv, D))
    assert np.max(np.abs(ref.attention(q, k, v) - _sdpa(q, k, v))) < 1e-12
    allowed = np.arange(nk)[None, :] <= (nk - nq + np.arange(nq))[:, None]
    assert np.max(np.abs(ref.attention(q, k, v, allowed) - _sdpa(q, k, v, allowed))) < 1e-12


def test_attention_special_cases():
    D = 8
    # one key: output is that value
    q = RNG.standard_normal((1, 2, D))
    k = RNG.standard_normal((1, 1, D))
    v = RNG.standard_normal((1, 1, D))
    assert np.allclose(ref.attention(q, k, v), np.repeat(v, 2, axis=1), atol=1e-15)
    # all keys equal: output is the mean of the values
    k = np.repeat(RNG.standard_normal((1, 1, D)), 9, axis=0)
    v = RNG.standard_normal((9, 1, D))
    assert np.allclose(ref.attention(q, k, v)[0, 0], v[:, 0].mean(axis=0), atol=1e-14)
    # hand value: D = 4, logits 4/sqrt(4) = 2 and 0 -> weights e^2/(1+e^2), 1/(1+e^2)
    q = np.array([[[2.0, 0, 0, 0]]])
    k = np.array([[[2.0, 0, 0, 0]], [[0.0, 0, 0, 0]]])
    v = np.array([[[1.0, 0, 0, 0]], [[0.0, 1, 0, 0]]])
    w1 = math.exp(2) / (1 + math.exp(2))
    assert np.allclose(ref.attention(q, k, v)[0, 0], [w1, 1 - w1, 0, 0], atol=1e-15)
    # GQA equals MHA over repeated kv heads
    q = RNG.standard_normal((5, 8, D))
    k = RNG.standard_normal((7, 2, D))
    v = RNG.standard_normal((7, 2, D))
    mha = ref.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    assert np.allclose(ref.attention(q, k, v), mha, atol=1e-14)


def test_softmax_rows_sum_to_one_via_constant_values():
    # with every value equal to 1 the output is the sum of the weights
    q = RNG.standard_normal((6, 4, 16))
    k = RNG.standard_normal((30, 2, 16)) * 3
    v = np.ones((30, 2, 16))
    assert np.allclose(ref.attention(q, k, v), 1.0, atol=1e-13)


# ---------------------------------------------------------------- argmax

def test_argmax_lowest_index_on_ties():
    z = RNG.integers(0, 4, size=(200, 13)).astype(float)
    got = ref.argmax_rows(z)
    for r in range(z.shape[0]):
        best = None
        for i in range(z.shape[1]):
            if best is None or z[r, i] > z[r, best]:
                best = i
        assert got[r] == best


def test_rel_err():
    assert ref.rel_err([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert ref.rel_err([1.0, 2.5], [1.0, 2.0]) == 0.25
