"""Pins of the prologue oracle (oracle/prologue.py) against special cases
with an independent definition: library functions (scipy's logistic),
shifts, causality, unit norms and closed forms of the gates."""
import numpy as np
import pytest
from scipy.special import expit

from oracle import prologue as PR


def make(B=2, N=9, H=2, d=4, r=3, K=4, seed=0, dm=None):
    rng = np.random.default_rng(seed)
    dm = dm or H * d
    C = 3 * H * d
    return dict(x=rng.standard_normal((B, N, dm)), W=rng.standard_normal((C + 4 * r, dm)) / np.sqrt(dm),
                w_conv=rng.standard_normal((C, K)), V=rng.standard_normal((4, H, r)), b=rng.standard_normal((4, H)),
                heads=H, d_head=d, rank=r)


def silu_ref(z):
    return z * expit(z)


def test_identity_tap_is_silu_of_the_projection_then_norm():
    a = make()
    K = a["w_conv"].shape[1]
    a["w_conv"][:] = 0.0
    a["w_conv"][:, K - 1] = 1.0            # the current token only
    q, k, v, _ = PR.prologue(**a)
    B, N, _ = a["x"].shape
    H, d = a["heads"], a["d_head"]
    P = a["x"] @ a["W"].T
    for i, (out, norm) in enumerate(((q, True), (k, True), (v, False))):
        want = silu_ref(P[..., i * H * d:(i + 1) * H * d]).reshape(B, N, H, d).transpose(0, 2, 1, 3)
        if norm:
            want = want / np.sqrt(np.sum(want ** 2, axis=-1, keepdims=True))
        np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-14)


def test_oldest_tap_shifts_by_k_minus_one():
    a = make(N=11)
    K = a["w_conv"].shape[1]
    ident = dict(a, w_conv=np.eye(1, K, K - 1).repeat(a["w_conv"].shape[0], 0))
    oldest = dict(a, w_conv=np.eye(1, K, 0).repeat(a["w_conv"].shape[0], 0))
    _, _, v1, _ = PR.prologue(**ident)
    _, _, v0, _ = PR.prologue(**oldest)
    np.testing.assert_allclose(v0[:, :, K - 1:], v1[:, :, :-(K - 1)], rtol=1e-13, atol=1e-14)
    # before the first token there is nothing: SiLU(0) = 0
    assert not v0[:, :, :K - 1].any()


def test_causal_with_a_receptive_field_of_k_tokens():
    a = make(N=12)
    K = a["w_conv"].shape[1]
    base = PR.prologue(**a)
    t0 = 5
    x2 = a["x"].copy()
    x2[:, t0] += 1.0
    pert = PR.prologue(**dict(a, x=x2))
    for i in range(3):
        np.testing.assert_array_equal(pert[i][:, :, :t0], base[i][:, :, :t0])
        np.testing.assert_array_equal(pert[i][:, :, t0 + K:], base[i][:, :, t0 + K:])
        assert np.abs(pert[i][:, :, t0:t0 + K] - base[i][:, :, t0:t0 + K]).min(axis=(0, 1, 3)).max() > 0
    # gates see only their own token
    np.testing.assert_array_equal(np.delete(pert[3], t0, axis=3), np.delete(base[3], t0, axis=3))


def test_sequences_are_independent():
    a = make(B=3)
    base = PR.prologue(**a)
    x2 = a["x"].copy()
    x2[1] = np.random.default_rng(9).standard_normal(x2[1].shape)
    pert = PR.prologue(**dict(a, x=x2))
    for i in range(4):
        ax = 1 if i == 3 else 0
        np.testing.assert_array_equal(np.take(pert[i], [0, 2], axis=ax), np.take(base[i], [0, 2], axis=ax))


def test_unit_norms():
    q, k, v, g = PR.prologue(**make(N=15))
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-13)
    assert np.abs(np.linalg.norm(v, axis=-1) - 1.0).max() > 1e-3
    assert ((g > 0) & (g < 1)).all()


def test_gate_closed_forms():
    a = make(r=2)
    H, d, r = a["heads"], a["d_head"], a["rank"]
    C = 3 * H * d
    a["V"][:] = 0.0
    _, _, _, g = PR.prologue(**a)
    for gi in range(4):
        np.testing.assert_allclose(g[gi], np.broadcast_to(expit(a["b"][gi])[None, :, None], g[gi].shape), rtol=1e-14)
    # U_g row j = e_j, V_g[h] = e_0: the gate is sigmoid(x[..., 0] + b)
    a = make(r=2)
    a["W"][C:] = 0.0
    for gi in range(4):
        a["W"][C + gi * r, 0] = 1.0
    a["V"][:] = 0.0
    a["V"][:, :, 0] = 1.0
    _, _, _, g = PR.prologue(**a)
    for gi in range(4):
        want = expit(a["x"][..., 0][:, None, :] + a["b"][gi][None, :, None])
        np.testing.assert_allclose(g[gi], want, rtol=1e-13)
