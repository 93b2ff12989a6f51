"""CPU checks of the GPU-vs-oracle comparison rules themselves: the score bound
is strict 1e-3 relative away from zero, its absolute floor only decides near
zero, and the floor ignores poisoned cache slots."""
import numpy as np
import pytest

import msa_synth
import parity_util as pu


def test_score_bound_is_strict_relative_away_from_zero():
    ref = np.array([[[5.0, -3.0, 0.2, -np.inf]]])
    floor = np.full((1, 1, 1), 4e-4)
    ok = ref.copy()
    ok[..., 0] *= 1 + 0.9e-3
    ok[..., 1] *= 1 - 0.9e-3
    ok[..., 2] += 3.9e-4                       # near zero: the floor decides
    worst = pu.check_scores(ok, ref, floor)
    assert 0.85e-3 < worst < 0.95e-3
    for i, bad in ((0, 5.0 * (1 + 1.1e-3)), (1, -3.0 * (1 - 1.2e-3)), (2, 0.2 + 4.1e-4)):
        b = ref.copy()
        b[0, 0, i] = bad
        with pytest.raises(AssertionError):
            pu.check_scores(b, ref, floor)
    b = ref.copy()
    b[0, 0, 3] = -1e30                        # -inf must stay -inf
    with pytest.raises(AssertionError):
        pu.check_scores(b, ref, floor)


def test_score_floor_is_small_and_ignores_poison():
    kw = dict(seed=17, ctx_lens=[700, 300], G=2, Hg=4, d_idx=128, k=2)
    clean = msa_synth.build_case("t", **kw)
    poisoned = msa_synth.build_case("t", poison=True, **kw)
    f0 = pu.score_floor(clean, [0, 1])
    f1 = pu.score_floor(poisoned, [0, 1])
    assert f0.shape == (2, 2, 1)
    np.testing.assert_array_equal(f0, f1)
    # N(0, 1) data: about 4e-4, an order of magnitude below 1e-3 of a typical
    # block score (about 5)
    assert np.all((f0 > 1e-4) & (f0 < 1e-3))
