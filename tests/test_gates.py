"""CPU checks of the parity gates themselves: each planted mistake in a result
(a NaN, a lost -inf, an element past the bound) must fail the gate, and the
unchanged result must pass it."""
import numpy as np
import pytest

from _cases import gate_f32, gate_lowp


def _ref(seed=0):
    rng = np.random.default_rng(seed)
    out = rng.standard_normal((4, 8, 64))
    lse = rng.standard_normal((4, 8)) * 3
    lse[1, 2] = -np.inf  # an empty key set
    out[1, 2] = 0.0
    return out, lse


@pytest.mark.parametrize("gate", ["f32", "lowp"])
def test_gate_passes_exact_result(gate):
    out, lse = _ref()
    if gate == "f32":
        gate_f32(out.copy(), out, "out")
        gate_f32(lse.copy(), lse, "lse")
    else:
        gate_lowp(out.copy(), out, "out", 2e-2)
        gate_lowp(lse.copy(), lse, "lse", 1e-3, norm=None)


@pytest.mark.parametrize("gate", ["f32", "lowp"])
@pytest.mark.parametrize("where", ["out", "lse"])
def test_gate_fails_on_nan(gate, where):
    out, lse = _ref()
    got_out, got_lse = out.copy(), lse.copy()
    (got_out if where == "out" else got_lse)[2, 3, ...] = np.nan
    got, ref = (got_out, out) if where == "out" else (got_lse, lse)
    with pytest.raises(AssertionError, match="NaN|non-finite"):
        if gate == "f32":
            gate_f32(got, ref, where)
        else:
            gate_lowp(got, ref, where, 2e-2 if where == "out" else 1e-3,
                      norm=1e-2 if where == "out" else None)


@pytest.mark.parametrize("gate", ["f32", "lowp"])
def test_gate_fails_on_lost_neg_inf(gate):
    _, lse = _ref()
    got = lse.copy()
    got[1, 2] = 0.0
    with pytest.raises(AssertionError, match="-inf"):
        if gate == "f32":
            gate_f32(got, lse, "lse")
        else:
            gate_lowp(got, lse, "lse", 1e-3, norm=None)


def test_gate_f32_fails_past_relative_bound():
    out, _ = _ref()
    got = out.copy()
    i = np.unravel_index(np.abs(out).argmax(), out.shape)
    got[i] *= 1 + 3e-5  # three times the 1e-5 relative tolerance on the largest element
    with pytest.raises(AssertionError, match="beyond fp32 gate"):
        gate_f32(got, out, "out")


def test_gate_lowp_fails_past_normalised_bound():
    out, _ = _ref()
    scale = np.abs(out).max()
    got = out.copy()
    got[0, 0, 0] += 2e-2 * scale  # within atol only if max|ref| were tiny; > 1e-2 max|ref|
    with pytest.raises(AssertionError):
        gate_lowp(got, out, "out", atol=1.0)
