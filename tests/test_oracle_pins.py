"""The oracle against its pins (CPU only)."""
import pytest

import oracle_checks as C


def test_bf16_rne_matches_torch():
    C.check_bf16_rne_vs_torch()


def test_int4_golden():
    C.check_int4_golden()


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("bf16_inputs", [False, True])
def test_int4_exact_replay(seed, bf16_inputs):
    C.check_int4_replay(seed=seed, bf16_inputs=bf16_inputs)


def test_int4_invariants():
    C.check_int4_invariants()


def test_fp4_golden():
    C.check_fp4_golden()


@pytest.mark.parametrize("seed", [0, 1])
def test_fp4_exact_replay(seed):
    C.check_fp4_replay(seed=seed)


def test_fp4_invariants():
    C.check_fp4_invariants()


def test_lambda():
    C.check_lambda()


def test_smoothing_balance():
    C.check_smoothing_balance()


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_reduction_to_plain_w4a4(mode):
    C.check_reduction_plain_w4a4(mode)


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_zero_residual(mode):
    C.check_zero_residual(mode)


def test_eckart_young():
    C.check_eckart_young()


@pytest.mark.parametrize("mode", ["int4", "fp4"])
def test_two_formulations(mode):
    C.check_two_formulations(mode)


@pytest.mark.parametrize("mode,seed,r", [("int4", 0, 2), ("int4", 1, 0), ("fp4", 0, 2), ("fp4", 2, 1)])
def test_pipeline_bruteforce(mode, seed, r):
    C.check_pipeline_bruteforce(mode=mode, seed=seed, r=r)


def test_rank_trend():
    C.check_rank_trend()
