"""Pins of the randomized-SVD oracle (CPU): Philox4x32-10 against the
known-answer vectors published with the Random123 library, CholeskyQR2
orthonormality, and the factors against the Eckart-Young optimum computed by
a full SVD; planted mistakes fail a pin."""
import numpy as np
import pytest

import oracle as O
import oracle.rsvd_oracle as R


@pytest.mark.parametrize("ctr,key,want", [
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
])
def test_philox_known_answers(ctr, key, want):
    assert O.philox4x32_10(ctr, key) == want


def test_rademacher_signs():
    om = O.rademacher(2000, 48, seed=7)
    assert set(np.unique(om)) == {-1.0, 1.0}
    assert abs(om.mean()) < 0.02
    assert np.array_equal(om, O.rademacher(2000, 48, seed=7))
    assert not np.array_equal(om, O.rademacher(2000, 48, seed=8))


def test_rademacher_blocks_past_128_columns():
    """Columns 128.. come from the next counter block: the first 128 columns
    do not depend on l, and column 128 + b is not column b again."""
    a = O.rademacher(300, 144, seed=11)
    assert np.array_equal(a[:, :128], O.rademacher(300, 128, seed=11))
    assert not np.array_equal(a[:, 128:], a[:, :16])
    w = O.philox4x32_10((5, 1, 0, 0), (11, 0))
    assert a[5, 128 + 9] == (-1.0 if (w[0] >> 9) & 1 else 1.0)


def test_eigenvector_signs_do_not_change_the_factors(monkeypatch):
    """The sign rule makes the factors independent of the signs the
    eigensolver returns."""
    A, _ = _decaying(200, 160, 2)
    L1, up, _ = O.rsvd_factors_f64(A, 16, seed=5)
    eigh = np.linalg.eigh

    def flipped(M):
        ev, V = eigh(M)
        return ev, V * np.where(np.arange(V.shape[1]) % 3 == 0, -1.0, 1.0)[None, :]

    monkeypatch.setattr(np.linalg, "eigh", flipped)
    L1b, upb, _ = O.rsvd_factors_f64(A, 16, seed=5)
    assert np.array_equal(L1, L1b) and np.array_equal(up, upb)
    # the largest component of every column of L1 (a positive multiple of
    # Q v) need not be positive, but each column pair keeps its product
    assert np.allclose(up @ L1.T, upb @ L1b.T)


def test_rank_128_sketch_wider_than_one_block():
    A, s = _decaying(400, 300, 6)
    r = 128
    L1, up, sv = O.rsvd_factors_f64(A, r, seed=2, power_iters=2)
    opt = np.sqrt(np.sum(s[r:] ** 2))
    assert np.linalg.norm(A - up @ L1.T) <= 1.10 * opt
    assert np.allclose(sv[:64], s[:64], rtol=1e-6)


def test_cholqr2_orthonormal():
    rng = np.random.default_rng(0)
    Y = rng.standard_normal((500, 40)) @ np.diag(np.logspace(0, 6, 40))
    Q = O.orth_cholqr2(Y)
    assert np.abs(Q.T @ Q - np.eye(40)).max() < 1e-10
    # same column space: Y = Q (Q^T Y)
    assert np.linalg.norm(Y - Q @ (Q.T @ Y)) <= 1e-9 * np.linalg.norm(Y)


def _decaying(N, K, seed):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((N, min(N, K))))
    V, _ = np.linalg.qr(rng.standard_normal((K, min(N, K))))
    s = 1.0 / (1.0 + np.arange(min(N, K))) ** 1.5
    return (U * s) @ V.T, s


def test_factors_reach_the_optimum():
    A, s = _decaying(300, 200, 1)
    r = 16
    L1, up, sv = O.rsvd_factors_f64(A, r, seed=3, power_iters=2)
    opt = np.sqrt(np.sum(s[r:] ** 2))                    # Eckart-Young
    err = np.linalg.norm(A - up @ L1.T)
    assert err <= 1.10 * opt
    assert np.allclose(sv, s[:r], rtol=1e-4)


def test_factors_of_an_exact_low_rank_matrix():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((120, 8)) @ rng.standard_normal((8, 96))
    L1, up, sv = O.rsvd_factors_f64(A, 8, seed=1, power_iters=0)
    # the sketch (l = 24 columns of a rank-8 range) is rank-deficient: the
    # shift keeps CholeskyQR defined and the range is still captured
    assert np.linalg.norm(A - up @ L1.T) <= 1e-5 * np.linalg.norm(A)


def test_zero_weight_gives_zero_factors():
    W = np.zeros((256, 128), np.uint16)
    ld, lu, s = O.rsvd_factors(W, np.ones(128, np.float32), 16, seed=1)
    assert not ld.any() and not lu.any() and not s.any()


def test_bf16_factors_shapes_and_product():
    rng = np.random.default_rng(5)
    W = O.f32_to_bf16((0.02 * rng.standard_normal((256, 128))).astype(np.float32))
    lam = np.exp(rng.uniform(-1, 1, 128)).astype(np.float32)
    ld, lu, s = O.rsvd_factors(W, lam, 16, seed=9)
    assert ld.shape == (16, 128) and lu.shape == (256, 16)
    What = O.bf16_to_f32(W).astype(np.float64) * lam.astype(np.float32).astype(np.float64)[None, :]
    P = O.bf16_to_f32(lu).astype(np.float64) @ O.bf16_to_f32(ld).astype(np.float64)
    _, sf, _ = np.linalg.svd(What)
    opt = np.sqrt(np.sum(sf[16:] ** 2))
    assert np.linalg.norm(What - P) <= 1.15 * opt


@pytest.mark.parametrize("bug", ["multiplier", "no_key_bump", "transpose_b"])
def test_mutations_fail_a_pin(bug, monkeypatch):
    if bug == "multiplier":
        monkeypatch.setattr(R, "_M0", 0xD2511F55)
        assert O.philox4x32_10((0, 0, 0, 0), (0, 0)) != (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)
    elif bug == "no_key_bump":
        monkeypatch.setattr(R, "_W0", 0)
        monkeypatch.setattr(R, "_W1", 0)
        assert O.philox4x32_10((0, 0, 0, 0), (0, 0)) != (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)
    else:
        A, s = _decaying(300, 200, 1)
        L1, up, _ = O.rsvd_factors_f64(A, 16, seed=3)
        opt = np.sqrt(np.sum(s[16:] ** 2))
        assert np.linalg.norm(A - up @ L1.T) <= 1.10 * opt
        # pairing the factors in the wrong order is far from the optimum
        assert not np.linalg.norm(A - (up[:, ::-1] @ L1.T)) <= 1.10 * opt
