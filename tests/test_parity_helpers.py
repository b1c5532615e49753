"""Host checks of the parity helpers the GPU tests rely on (tests/q3_testutil.py): the bar is
applied as stated, a tensor compared in pieces gives exactly the figures of one comparison of
the whole, and the bf16-reference diagnostic separates output rounding from other error."""
import numpy as np
import pytest

import synth
from q3_testutil import RECORDS, ParityAccumulator, parity


def _bf16(x):
    return synth.bf16_to_f32(synth.f32_to_bf16(np.asarray(x, np.float32))).astype(np.float64)


def test_pieces_equal_the_whole():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((40, 33))
    got = ref + 1e-3 * rng.standard_normal(ref.shape)
    parity(got, ref, "whole", stored_bf16=True)
    whole = RECORDS[-1]
    acc = ParityAccumulator("pieces", stored_bf16=True)
    for r0 in range(0, 40, 7):  # ragged last piece
        acc.add(got[r0:r0 + 7], ref[r0:r0 + 7])
    acc.check()
    pieces = RECORDS[-1]
    for k in ("n", "max_abs", "max_abs_vs_bf16_ref"):
        assert pieces[k] == whole[k], k
    for k in ("rms", "max_abs_bar", "mean_rel"):
        assert pieces[k] == pytest.approx(whole[k], rel=1e-12), k


def test_output_rounding_alone_reads_zero_against_the_rounded_reference():
    rng = np.random.default_rng(6)
    ref = rng.standard_normal(1000) * 3.0
    got = _bf16(ref)
    parity(got, ref, "rounded", stored_bf16=True)
    rec = RECORDS[-1]
    assert rec["max_abs_vs_bf16_ref"] == 0.0
    # half an ulp of the largest magnitude bounds the error against the exact reference
    assert 0.0 < rec["max_abs"] <= np.abs(ref).max() * 2.0 ** -8


def test_the_bar_is_enforced():
    ref = np.linspace(-1.0, 1.0, 101)
    rms = float(np.sqrt(np.mean(ref * ref)))
    near = ref.copy()
    near[50] += 0.99 * 2e-2 * rms  # one element just inside the max-abs bar
    parity(near, ref, "inside")
    far = ref.copy()
    far[50] += 1.01 * 2e-2 * rms  # one element just past it
    with pytest.raises(AssertionError):
        parity(far, ref, "outside")
    drift = ref * (1.0 + 6e-3)  # every element off by 0.6%: mean relative error past 5e-3
    with pytest.raises(AssertionError):
        parity(drift, ref, "drift")
    acc = ParityAccumulator("outside in pieces")
    acc.add(far[:50], ref[:50])
    acc.add(far[50:], ref[50:])
    with pytest.raises(AssertionError):
        acc.check()
    with pytest.raises(AssertionError):
        parity(np.full(3, np.nan), np.ones(3), "non-finite")
