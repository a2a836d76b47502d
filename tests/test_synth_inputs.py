"""The seeded input generator: determinism, row independence, pinned checksums and the statistics
of the synthetic workloads (stand-ins for the LLM weight matrices the QAM-W paper evaluates)."""
import hashlib

import numpy as np
import pytest


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def test_rows_are_independent_of_the_slice(synth):
    m = synth.config(1).matrices[0]
    full = m.weights(0, 40)
    np.testing.assert_array_equal(m.weights(17, 9), full[17:26])


def test_pinned_checksums(synth):
    c1 = synth.config(1)
    m = c1.matrices[0]
    got = {
        "cfg1_rows0_8": _sha(m.weights(0, 8)),
        "cfg1_scale": _sha(m.channel_scale()),
        "cfg1_points_4096": _sha(synth.points(c1.seed, 4, 4096)),
        "cfg0_rows": _sha(synth.config(0).matrices[0].weights()),
    }
    assert got == PINNED, got


PINNED = {'cfg1_rows0_8': '918e5a424c249500', 'cfg1_scale': '75b452ba08055122', 'cfg1_points_4096': '42da9f1667686020', 'cfg0_rows': '261e4d3a9b9efbfc'}


def test_statistics(synth):
    c = synth.config(1)
    m = c.matrices[0]
    assert (m.d_out, m.d_in, m.n_outlier) == (4096, 4096, 41)
    w = synth.bf16_bits_to_f32(m.weights(0, 256)).astype(np.float64)
    cols = m.outlier_columns()
    normal = np.setdiff1d(np.arange(m.d_in), cols)
    # Student-t(5) x 0.015: variance 5/3 * 0.015^2, outlier columns x10
    assert np.std(w[:, normal]) == pytest.approx(0.015 * np.sqrt(5 / 3), rel=0.03)
    assert np.std(w[:, cols]) == pytest.approx(0.15 * np.sqrt(5 / 3), rel=0.15)
    s = m.channel_scale()
    assert s.min() >= 0.1 and s.dtype == np.float32
    p = synth.points(c.seed, 4, 1 << 16).astype(np.float64)
    assert np.abs(p.mean(0)).max() < 0.02 and np.abs(p.std(0) - 1).max() < 0.02
    assert abs(np.corrcoef(p.T)[0, 1]) < 0.02
    assert [x.n_outlier for x in synth.config(2).matrices] == [20, 55]
    assert sum(x.d_out * x.d_in for x in synth.config(4).matrices) == 12687769600


def test_config_shapes(synth):
    c3 = synth.config(3)
    assert [(x.d_out, x.d_in) for x in c3.matrices] == [(5120, 5120)] * 4 + [(13824, 5120)] * 2 + [(5120, 13824)]
    assert c3.bits == [11, 7] and c3.block == 128
    assert synth.config(0).fixed_sigma == 0.125 and synth.config(0).bits == [8]
