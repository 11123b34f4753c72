"""The oracle against facts fixed independently of it: the pages' printed
figures and rules (golden fixtures), closed forms, exact rational arithmetic
with the pages' error bound, brute force on tiny inputs, and library routines
(numpy expansion + matmul, Python sorting) on an independent route."""
import numpy as np
import pytest

import oracle
from tests import _independent as I
from tests import _pins as P


@pytest.fixture(scope="module")
def O():
    return oracle.Oracle()


@pytest.mark.parametrize("check", P.ALL, ids=[c.__name__ for c in P.ALL])
def test_pin(O, check):
    check(O)


def test_census_matches_pages():
    """Census figures the pages print, recomputed from the format: one expert
    is 3 matrices of 7168x1536 at 0.5 + 1/32 bytes per weight."""
    c = I.read_census()
    hidden, inter = 7168, 1536
    params = 3 * hidden * inter
    assert params == c["params_per_expert"]
    bytes_per_weight = 0.5 + 1.0 / 32
    assert bytes_per_weight == c["bytes_per_weight"]
    packed = params // 2 + params // 32
    assert packed == c["bytes_per_expert"]
    # printed to 3 decimals (the page rounds from 17.55 MB per expert)
    assert abs(c["routed_experts_total"] * packed / 1e12 - c["routed_total_TB"]) <= 1e-3
    assert round(c["experts_per_token"] * packed / 1e9, 2) == c["packed_GB_per_token"]
    assert round(params * 4 / 1e6) == c["fp32_MB_per_expert"]
    assert int(c["experts_per_token"] * params * 4 / 1e9) == c["fp32_GB_per_token"]
    assert round(4 / bytes_per_weight, 1) == c["fewer_bytes_ratio"]
    assert hidden == c["hidden"]


def test_generated_expert_bytes_match_census():
    import gen
    E = gen.expert(0, 2, 0, 7168, 1536)
    total = sum(a.nbytes for m in ("gate", "up", "down") for a in E[m])
    assert total == I.read_census()["bytes_per_expert"]


def test_refusals(O):
    nib = np.zeros((2, 24), np.uint8)
    sc = np.zeros((2, 2), np.uint8)
    with pytest.raises(oracle.OracleError):
        O.gemv(nib, sc, np.zeros(48), group=16)  # only group 32 is described
    with pytest.raises(oracle.OracleError):
        O.topk(np.zeros(4), 5)  # k > n
