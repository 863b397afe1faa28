"""CPU pins of the FP64 oracle (no GPU): every check encodes a fact that does
not come from the oracle itself (dense products, exact rationals, closed
forms, invariants)."""

import pytest

import oracle_pins as P
from oracle import abc_bwd_ref, abc_ref, chunked_ref, gdr_bwd_ref, gdr_ref, kda_ref


@pytest.mark.parametrize("check", P.GDR_CHECKS, ids=lambda f: f.__name__)
def test_gdr_oracle_pin(check):
    check(gdr_ref)


def test_chunked_form_equals_token_recurrence():
    P.check_chunk_algebra(gdr_ref, chunked_ref)


@pytest.mark.parametrize("check", P.ABC_CHECKS, ids=lambda f: f.__name__)
def test_abc_oracle_pin(check):
    check(abc_ref)


@pytest.mark.parametrize("check", P.BWD_CHECKS, ids=lambda f: f.__name__)
def test_backward_oracle_pin(check):
    P.run_bwd_check(check, gdr_bwd_ref, gdr_ref, chunked_ref)


@pytest.mark.parametrize("check", P.ABC_READ_CHECKS, ids=lambda f: f.__name__)
def test_abc_read_oracle_pin(check):
    check(abc_ref)


@pytest.mark.parametrize("check", P.ABC_BWD_CHECKS, ids=lambda f: f.__name__)
def test_abc_backward_oracle_pin(check):
    P.run_abc_bwd_check(check, abc_bwd_ref, abc_ref)


@pytest.mark.parametrize("check", P.KDA_CHECKS, ids=lambda f: f.__name__)
def test_kda_oracle_pin(check):
    check(kda_ref)


def test_kda_reduces_to_scalar_decay():
    P.check_kda_scalar_reduction(kda_ref, gdr_ref)


def test_kda_chunk_form_equals_token_recurrence():
    P.check_kda_chunk_algebra(kda_ref)
