"""The GPU tests' checkers, on the CPU: the whole-output projection check
(helpers.freivalds) and the parity rule (helpers.parity) must pass a correct
result and fail one with an unwritten (NaN-filled) or wrong block of C."""
import numpy as np
import pytest

import helpers
import oracle
from dense_half_precision_amd import inputs


@pytest.fixture(scope="module")
def tn_case():
    oracle.build(0, force=False)
    M = N = K = 256
    A = inputs.draw((M, K), "f16", "uniform", 7001)
    Bt = inputs.draw((N, K), "f16", "uniform", 7002)
    return A, Bt, oracle.hgemm("tn", "f16", A, Bt)


def test_freivalds_passes_correct_output(tn_case):
    A, Bt, C = tn_case
    helpers.freivalds(C, A, Bt, "tn", "f16")
    helpers.freivalds(C.T.copy(), Bt, A, "tn", "f16")


@pytest.mark.parametrize("fill", [0x7E00, 0xFE00, 0x7C00])
def test_freivalds_fails_on_unwritten_block(tn_case, fill):
    """A 16 x 16 block left at the output buffer's NaN (or inf) fill."""
    A, Bt, C = tn_case
    bad = C.copy()
    bad[96:112, 32:48] = fill
    with pytest.raises(AssertionError, match="non-finite"):
        helpers.freivalds(bad, A, Bt, "tn", "f16")


def test_freivalds_fails_on_wrong_block(tn_case):
    """A finite but wrong 16 x 16 block (a tile computed from the wrong k range
    would look like this)."""
    A, Bt, C = tn_case
    bad = C.copy()
    vals = helpers.decode(bad[96:112, 32:48], "f16") * 0.5
    bad[96:112, 32:48] = vals.astype(np.float16).view(np.uint16)
    with pytest.raises(AssertionError, match="Freivalds check failed"):
        helpers.freivalds(bad, A, Bt, "tn", "f16")


def test_parity_rule_rejects_nan_and_wrong(tn_case):
    _, _, C = tn_case
    helpers.parity(C, C, "f16", "identical")
    nan = C.copy()
    nan[5, 7] = 0x7E00
    with pytest.raises(AssertionError, match="non-finite"):
        helpers.parity(nan, C, "f16", "nan")
    off = C.copy()
    off[5, 7] ^= 0x4000  # flips an exponent bit: far outside the tolerance
    with pytest.raises(AssertionError):
        helpers.parity(off, C, "f16", "wrong")
