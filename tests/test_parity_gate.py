"""The O gate of the GPU parity tests, on hand-made arrays (CPU only).

Below |O| = 2 the raw error must stay within 1e-2; from |O| = 2 on, where the bf16
rounding of the output alone takes 0.0078 (|O| in [2, 4)) or more of it, the 1e-2
applies beyond that half ulp. LSE and the yardstick gate are plain comparisons."""
import numpy as np
import pytest

from parity_util import _merge, assert_parity, bf16_half_ulp, o_errors


def err_for(o, O_ref, dlse=0.0, e_unf=1.0):
    e = o_errors(np.array(o, dtype=np.float64), np.array(O_ref, dtype=np.float64))
    e.update(max_dLSE=dlse, finite=True, E_unf=e_unf, rows_checked=1)
    return e


def test_half_ulp_values():
    np.testing.assert_array_equal(bf16_half_ulp(np.array([1.0, 1.99, 2.0, 3.5, 4.0, 7.9, 0.5])),
                                  [2 ** -8, 2 ** -8, 2 ** -7, 2 ** -7, 2 ** -6, 2 ** -6, 2 ** -9])


def test_small_values_are_gated_raw():
    assert_parity(err_for([0.5 + 0.0099], [0.5]), "ok")
    with pytest.raises(AssertionError):
        assert_parity(err_for([0.5 + 0.0101], [0.5]), "raw 1e-2 exceeded")
    with pytest.raises(AssertionError):
        assert_parity(err_for([1.99 - 0.0101], [1.99]), "raw 1e-2 exceeded just below 2")


def test_wide_values_get_the_rounding_allowance():
    # |O| = 5: half an ulp is 2^-6 = 0.0156; 0.02 is 0.0044 beyond it
    e = err_for([5.02], [5.0])
    assert e["n_wide"] == 1 and e["n_over_tol"] == 1
    assert_parity(e, "wide, within")
    with pytest.raises(AssertionError):
        assert_parity(err_for([5.0 + 0.0157 + 0.0101], [5.0]), "wide, beyond")
    # |O| = 3: half an ulp is 2^-8 ... 2^-7 = 0.0078; 0.0105 is 0.0027 beyond it, and counted
    e = err_for([3.0 + 0.0105], [3.0])
    assert e["n_over_tol"] == 1 and e["max_dO"] > 0.01
    assert_parity(e, "[2, 4): within")
    # the size is the larger of the two magnitudes: exact 1.999 computed as 2.0078
    assert err_for([2.0078125], [1.999])["n_wide"] == 1


def test_lse_and_yardstick_gates():
    with pytest.raises(AssertionError):
        assert_parity(err_for([1.0], [1.0], dlse=1.1e-3), "lse")
    with pytest.raises(AssertionError):
        assert_parity(err_for([1.003], [1.0], e_unf=0.001), "2 x E_unf")
    assert_parity(err_for([1.003], [1.0], e_unf=0.0016), "2 x E_unf ok")


def test_merge_keeps_worst_and_counts():
    a = err_for([1.001, 5.01], [1.0, 5.0])
    b = err_for([0.2], [0.2 + 0.004])
    m = _merge(a, b)
    assert m["n_elements"] == 3 and m["n_wide"] == 1 and m["max_dO_wide_beyond_rounding"] < 0
    assert m["max_dO_narrow"] == pytest.approx(0.004)
    assert m["max_dO"] == pytest.approx(0.01)
