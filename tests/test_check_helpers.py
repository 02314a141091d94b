"""CPU checks of the comparison helpers the GPU tests rely on."""
import numpy as np

from kda_check import PerHeadSeqErr, rel_err_per_head


def test_per_head_sequence_error_equals_whole_sequence_ratio():
    """Adding a decode run step by step gives, per head, max|got - ref| over all of
    the head's outputs divided by their RMS: the prefill definition applied to
    the head's output sequence."""
    rng = np.random.default_rng(0)
    steps, heads, dv = 7, 5, 16
    ref = rng.normal(size=(steps, heads, dv)) * rng.uniform(0.1, 10, size=(1, heads, 1))
    got = ref + rng.normal(scale=1e-3, size=ref.shape)
    acc = PerHeadSeqErr()
    for t in range(steps):
        acc.add(got[t], ref[t])
    whole = rel_err_per_head(got.transpose(1, 0, 2), ref.transpose(1, 0, 2))
    assert abs(acc.value() - whole) <= 1e-12 * whole
    # a head's error is judged against its own scale, not the step's
    got2 = ref.copy()
    got2[:, 0] += 0.05 * np.sqrt(np.mean(ref[:, 0] ** 2))
    acc2 = PerHeadSeqErr()
    for t in range(steps):
        acc2.add(got2[t], ref[t])
    assert abs(acc2.value() - 0.05) < 1e-9


def test_per_head_sequence_error_flags_non_finite():
    acc = PerHeadSeqErr()
    acc.add(np.array([[np.nan, 0.0]]), np.array([[1.0, 1.0]]))
    assert acc.value() == float("inf")
