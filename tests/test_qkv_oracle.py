"""Pins of the Q/K RMSNorm + RoPE oracle (CPU): closed forms and invariants
that a dropped term, a wrong sign or a swapped pair element breaks."""
import numpy as np
import pytest

import oracle as O
import oracle.qkv_oracle as QO


def _inputs(M=5, H=3, seed=0):
    rng = np.random.default_rng(seed)
    Y = rng.standard_normal((M, 3 * H * 128)) * 3.0
    qs = rng.uniform(0.5, 1.5, 128)
    ks = rng.uniform(0.5, 1.5, 128)
    ang = rng.uniform(-np.pi, np.pi, (M, 64))
    return Y, qs, ks, np.cos(ang), np.sin(ang), ang


def test_rmsnorm_unit_scale_has_unit_rms():
    Y, _, _, _, _, _ = _inputs()
    Z = O.rms_norm_heads(Y[:, :384], np.ones(128), eps=0.0)
    rms = np.sqrt(np.mean(Z.reshape(5, 3, 128) ** 2, axis=2))
    assert np.allclose(rms, 1.0, rtol=1e-12)
    # scale-invariant: a head scaled by c gives the same output
    Z2 = O.rms_norm_heads(7.5 * Y[:, :384], np.ones(128), eps=0.0)
    assert np.allclose(Z, Z2, rtol=1e-12)


def test_rmsnorm_one_head_by_hand():
    x = np.arange(1, 129, dtype=np.float64)[None, :]
    s = np.full(128, 2.0)
    want = x / np.sqrt(np.sum(x * x) / 128 + 1e-6) * 2.0
    assert np.allclose(O.rms_norm_heads(x, s, 1e-6), want, rtol=1e-14)


def test_rope_is_a_rotation_of_each_pair():
    Y, _, _, c, s, ang = _inputs()
    X = Y[:, :384]
    R = O.rope_pairs(X, c, s)
    p = X.reshape(5, 3, 64, 2)
    r = R.reshape(5, 3, 64, 2)
    # norms of the pairs are kept, and the angle grows by ang[m][i]
    assert np.allclose(np.hypot(p[..., 0], p[..., 1]), np.hypot(r[..., 0], r[..., 1]), rtol=1e-12)
    d = np.angle(r[..., 0] + 1j * r[..., 1]) - np.angle(p[..., 0] + 1j * p[..., 1])
    d = (d - ang[:, None, :] + np.pi) % (2 * np.pi) - np.pi
    assert np.abs(d).max() < 1e-9
    # zero angles are the identity, and rotating back undoes it
    assert np.allclose(O.rope_pairs(X, np.ones_like(c), np.zeros_like(s)), X)
    assert np.allclose(O.rope_pairs(R, c, -s), X, rtol=1e-12, atol=1e-12)


def test_qk_norm_rope_pieces_and_v_passthrough():
    Y, qs, ks, c, s, _ = _inputs(seed=3)
    Q, K, V = O.qk_norm_rope(Y, 3, qs, ks, c, s, eps=1e-6)
    assert np.array_equal(V, Y[:, 768:])
    assert np.allclose(Q, O.rope_pairs(O.rms_norm_heads(Y[:, :384], qs, 1e-6), c, s))
    assert np.allclose(K, O.rope_pairs(O.rms_norm_heads(Y[:, 384:768], ks, 1e-6), c, s))
    # Q does not depend on K's scale and vice versa
    Q2, K2, _ = O.qk_norm_rope(Y, 3, qs, 2 * ks, c, s)
    assert np.array_equal(Q, Q2) and np.allclose(K2, 2 * K)


@pytest.mark.parametrize("bug", ["sin_sign", "pair_swap", "mean_vs_sum"])
def test_mutations_fail_a_pin(bug, monkeypatch):
    Y, qs, ks, c, s, ang = _inputs(seed=7)
    X = Y[:, :384]
    if bug == "sin_sign":
        bad = O.rope_pairs(X, c, -s)
        r = bad.reshape(5, 3, 64, 2)
        p = X.reshape(5, 3, 64, 2)
        d = np.angle(r[..., 0] + 1j * r[..., 1]) - np.angle(p[..., 0] + 1j * p[..., 1])
        d = (d - ang[:, None, :] + np.pi) % (2 * np.pi) - np.pi
        assert np.abs(d).max() > 1e-3
    elif bug == "pair_swap":
        bad = O.rope_pairs(X.reshape(5, 3, 64, 2)[..., ::-1].reshape(5, 384), c, s)
        assert not np.allclose(bad, O.rope_pairs(X, c, s))
    else:
        monkeypatch.setattr(QO.np, "mean", np.sum)
        Z = QO.rms_norm_heads(X, np.ones(128), eps=0.0)
        monkeypatch.undo()
        rms = np.sqrt(np.mean(Z.reshape(5, 3, 128) ** 2, axis=2))
        assert not np.allclose(rms, 1.0)
