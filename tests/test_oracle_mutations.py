"""Plant plausible mistakes in the oracle (on the CPU) and check that at
least one pin catches each of them."""
import numpy as np
import pytest

import oracle.svdq_oracle as O
import oracle_checks as C

ALL = [
    C.check_int4_golden, C.check_fp4_golden,
    lambda: C.check_int4_replay(0), lambda: C.check_fp4_replay(0),
    C.check_int4_invariants, C.check_fp4_invariants, C.check_lambda,
    C.check_smoothing_balance,
    lambda: C.check_reduction_plain_w4a4("int4"), lambda: C.check_reduction_plain_w4a4("fp4"),
    lambda: C.check_zero_residual("int4"), lambda: C.check_zero_residual("fp4"),
    C.check_eckart_young,
    lambda: C.check_pipeline_bruteforce("int4", 0), lambda: C.check_pipeline_bruteforce("fp4", 0),
]


def _some_check_fails():
    for chk in ALL:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


_orig_q4 = O.quantize_int4
_orig_fp4 = O.quantize_fp4
_orig_res = O.residual
_orig_lr = O.lowrank_factors


def _q4_div8(V):
    V = np.asarray(V, np.float32)
    rows, K = V.shape
    Vg = V.reshape(rows, K // 64, 64)
    s = (np.abs(Vg).max(axis=2) / np.float32(8)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[:, :, None] > 0, np.clip(np.rint(Vg / np.where(s > 0, s, 1)[:, :, None]), -8, 7), 0)
    return q.astype(np.int8).reshape(rows, K), s


def _q4_half_up(V):
    V = np.asarray(V, np.float32)
    rows, K = V.shape
    Vg = V.reshape(rows, K // 64, 64)
    s = (np.abs(Vg).max(axis=2) / np.float32(7)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (Vg / np.where(s > 0, s, 1)[:, :, None]).astype(np.float32)
    q = np.where(s[:, :, None] > 0, np.clip(np.sign(quot) * np.floor(np.abs(quot) + 0.5), -8, 7), 0)
    return q.astype(np.int8).reshape(rows, K), s


def _fp4_exp_minus1(V, chunk_rows=256):
    """Scale exponent floor(log2 a) - 1 instead of - 2 (block max lands in [2, 4))."""
    V = np.asarray(V, np.float32)
    rows, K = V.shape
    Vb = V.reshape(rows, K // 32, 32).astype(np.float64)
    a = np.abs(Vb).max(axis=2)
    _, ex = np.frexp(a)
    e = np.where(a > 0, np.clip(ex - 1 - 1, -127, 127), -127).astype(np.int64)
    y = np.ldexp(Vb, -e[:, :, None])
    return O._e2m1_code(y).reshape(rows, K), (e + 127).astype(np.uint8)


def _res_plus(W_hat, L1, L2):
    R = _orig_res(W_hat, L1, L2)
    return (2 * np.asarray(W_hat, np.float32) - R).astype(np.float32)   # W_hat + acc


def _lr_unbalanced(W_hat, r):
    L1, L2, S = _orig_lr(W_hat, r)
    if r == 0:
        return L1, L2, S
    U, S2, Vt = np.linalg.svd(np.asarray(W_hat, np.float64).T, full_matrices=False)
    return (O.f32_to_bf16((U[:, :r] * S2[:r]).astype(np.float32)),
            O.f32_to_bf16(Vt[:r].astype(np.float32)), S2)


def _lam_inverted(X, W):
    return (1.0 / _orig_lam(X, W)).astype(np.float32)


_orig_lam = O.calibrate_lambda
_orig_smooth = O.smooth_act
_orig_pack = O.pack_nibbles
_orig_fwd = O.forward


def _smooth_mul(X, lam):
    q = (O.bf16_to_f32(X) * np.asarray(lam, np.float32)[None, :]).astype(np.float32)
    return O.f32_to_bf16(q)


def _pack_swapped(codes):
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[:, 1::2] | (c[:, 0::2] << 4)).astype(np.uint8)


MUTATIONS = {
    "int4 scale absmax/8": ("quantize_int4", _q4_div8),
    "int4 rounds half away from zero": ("quantize_int4", _q4_half_up),
    "fp4 scale exponent off by one": ("quantize_fp4", _fp4_exp_minus1),
    "residual adds the low-rank part": ("residual", _res_plus),
    "unbalanced singular-value split": ("lowrank_factors", _lr_unbalanced),
    "lambda inverted": ("calibrate_lambda", _lam_inverted),
    "activations multiplied by lambda": ("smooth_act", _smooth_mul),
    "nibble order swapped": ("pack_nibbles", _pack_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    assert _some_check_fails(), f"no pin caught: {name}"


def test_dropped_bias_is_caught(monkeypatch):
    def fwd(xc, xs, T, wc, ws, L2, bias, mode):
        return _orig_fwd(xc, xs, T, wc, ws, L2, None, mode)
    monkeypatch.setattr(O, "forward", fwd)
    assert _some_check_fails()


def test_dropped_lowrank_branch_is_caught(monkeypatch):
    def fwd(xc, xs, T, wc, ws, L2, bias, mode):
        return _orig_fwd(xc, xs, None, wc, ws, L2, bias, mode)
    monkeypatch.setattr(O, "forward", fwd)
    assert _some_check_fails()
