"""The planted rising-key workloads really drive an online softmax with a
lazily moved reference (slack 8 log2 units, 32-token tiles) through its
rescale path: most rows move their reference at least twice, some by more
than 16 log2 units. Checked from float64 scores on the CPU, so the GPU tests
that use these workloads are known to exercise the rescale."""
import pytest

import rescale_util as R


@pytest.mark.parametrize("name", sorted(R.SPECS))
def test_planted_keys_cross_the_slack(name):
    wl = R.rising_workload(name)
    frac, big = R.check_crossings(wl)
    assert frac >= 0.6, f"{name}: only {frac:.2f} of rows move their reference twice"
    assert big >= 16.0, f"{name}: largest move {big:.1f} log2 units"
