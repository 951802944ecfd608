"""The oracle's one-stage dispatch predicate against the hand-derived cases in
tests/golden/one_stage_cases.txt (each derived from the rule's printed
constants), plus the configurations of the five workloads."""
import pytest

import oracle
from golden_cases import one_stage_cases
from tp_all_reduce_amd import workloads

CASES = one_stage_cases()


def test_fixture_is_not_empty():
    assert len(CASES) >= 20


@pytest.mark.parametrize("W,numel,hidden,dtype,fc,expected,note", CASES,
                         ids=[c[-1] or str(i) for i, c in enumerate(CASES)])
def test_one_stage_case(W, numel, hidden, dtype, fc, expected, note):
    assert oracle.one_stage(W, numel, hidden, dtype, fc) == bool(expected)


def test_workload_dispatch():
    # c1 -> one stage; c2 -> one stage up to T=31 only; c3/c4 -> never
    c1, c2, c3, c4 = (workloads.WORKLOADS[k] for k in ("c1", "c2", "c3", "c4"))
    assert oracle.one_stage(c1.W, 8 * c1.H, c1.H, oracle.BF16)
    got = {T: oracle.one_stage(c2.W, T * c2.H, c2.H, oracle.BF16) for T in c2.Ts}
    assert got == {1: True, 2: True, 4: True, 8: True, 16: True, 21: True, 22: True,
                   32: False, 64: False, 80: False}
    assert not any(oracle.one_stage(c3.W, T * c3.H, c3.H, oracle.BF16) for T in c3.Ts)
    assert not oracle.one_stage(c4.W, 256 * c4.H, c4.H, oracle.BF16)
