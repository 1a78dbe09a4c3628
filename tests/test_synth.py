"""Seeded input generators: determinism and row-range regeneration.  CPU only."""
import numpy as np

import synth


def test_weight_rows_match_full_across_blocks():
    K, N = 64, 2 * synth.ROW_BLOCK + 100
    full = synth.weight(9, K, N, outliers=True)
    for r0, r1 in [(0, 5), (synth.ROW_BLOCK - 3, synth.ROW_BLOCK + 7), (N - 50, N), (17, 17)]:
        assert np.array_equal(synth.weight_rows(9, K, N, r0, r1, outliers=True), full[r0:r1])


def test_deterministic_and_distribution():
    a = synth.weight(2, 512, 256)
    assert np.array_equal(a, synth.weight(2, 512, 256))
    assert abs(float(a.std()) - 0.02) < 0.001 and abs(float(a.mean())) < 0.001
    b = synth.weight(2, 512, 256, outliers=True)
    frac = np.mean(np.abs(b) > 0.1)        # |w| > 5 sigma: essentially only outliers
    assert 0.004 < frac < 0.012
    x = synth.activation(2, 4096, 4)
    assert x.dtype == np.uint16 and np.array_equal(x, synth.activation(2, 4096, 4))
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(xf.std()) - 1.0) < 0.05


def test_structured_inputs():
    x = synth.one_hot_activation(256, [0, 255])
    assert x[0, 0] == 0x3F80 and x[1, 255] == 0x3F80 and int(x.astype(bool).sum()) == 2
    eye = synth.identity_activation(16)
    assert np.array_equal(eye != 0, np.eye(16, dtype=bool))
