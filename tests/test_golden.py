"""The oracle still reproduces its committed regression record."""
import numpy as np

from golden import make_golden


def test_oracle_matches_golden_record():
    rec = make_golden.load()
    inp, out, pool = make_golden.compute()
    np.testing.assert_allclose(out.ravel(), rec["out"], rtol=0, atol=1e-15)
    for s in inp.state_idx:
        np.testing.assert_array_equal(pool[s, 1, :4].ravel(),
                                      rec[f"slot{s}_h1_rows0to3"].astype(np.float32))
        assert abs(pool[s].astype(np.float64).sum() - rec[f"slot{s}_sum"][0]) <= 1e-12
