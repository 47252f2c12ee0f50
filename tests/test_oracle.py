"""The fp64 oracle against the pages' worked examples, closed forms, invariants
and library routines (CPU only)."""
import math

import pytest

import oracle
import oracle_checks as oc
import pagealgos as pa


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(lib, check):
    check(lib)


def test_online_trace_matches_printed_example():
    # the element-by-element recurrence used by the checks reproduces the
    # printed running state of the first page's worked example
    g = pa.read_golden(oc.os.path.join(oc.GOLDEN, "softmax_worked_example.txt"))
    tol = 0.5 * 10 ** (-int(g["decimals"][0][0])) + 1e-12
    x = [float(t) for t in g["x"][0]]
    _, states = pa.scan(x)
    assert [s[0] for s in states] == [float(t) for t in g["online_m"][0]]
    assert all(abs(s[1] - float(b)) <= tol for s, b in zip(states, g["online_d"][0]))


def test_tile_recurrence_equals_scalar():
    # four elements in two tiles of two, as the first page suggests
    x = [1.0, 3.0, 2.0, 5.0]
    (m1, l1), _ = pa.scan(x)
    m2, l2 = pa.fold_left(pa.segments(x, [2, 2]))
    assert m1 == m2 and abs(l1 - l2) <= 1e-15
    assert abs(pa.lse((m1, l1)) - (5 + math.log(l1))) == 0
