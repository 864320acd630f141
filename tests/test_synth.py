"""Host checks of the seeded input generators and the parity helper (CPU only)."""

import numpy as np

import synth
from tests import parity


def test_tiny_recipe_is_seed_zero():
    w, x = synth.tiny_fp4_inputs()
    rng = np.random.default_rng(0)
    w2 = rng.normal(0, 0.02, (256, 512)).astype(np.float32)
    assert np.array_equal(w, w2) and x.shape == (1, 512) and x.dtype == np.uint16


def test_weight_rows_match_full_matrix():
    sid, n, k = 4, 9000, 64
    full = synth.weights(sid, n, k, layer=2)
    rows = synth.sample_rows(n, 50)
    assert rows[0] == 0 and rows[-1] == n - 1
    assert np.array_equal(synth.weight_rows(sid, n, k, rows, layer=2), full[rows])
    assert np.array_equal(full, synth.weights(sid, n, k, layer=2, threads=1))


def test_weights_distribution():
    w = synth.weights(1, 4096, 256)
    assert abs(w.std() - 0.02) < 2e-4 and abs(w.mean()) < 2e-4


def test_activations_are_bf16_of_normal():
    x = synth.activations(3, 4, 1024)
    assert x.shape == (4, 1024) and x.dtype == np.uint16
    v = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(v.std() - 1.0) < 0.05
    assert not np.array_equal(x[0], x[1])


def test_parity_helper_guard():
    y_ref = np.array([1.0, 1e-9, -2.0])
    a_ref = np.array([1.0, 100.0, 2.0])
    ok = parity.report(y_ref * (1 + 5e-4), y_ref, a_ref)
    assert ok["ok"]
    bad = parity.report(y_ref * (1 + 2e-3), y_ref, a_ref)
    assert not bad["ok"]
    # the cancelling element is judged against 2**-12 * A
    r = parity.report(np.array([1.0, 1e-9 + 1e-5, -2.0]), y_ref, a_ref)
    assert r["ok"] and r["guarded_elems"] == 1
    assert not parity.report(np.array([np.nan, 0, 0]), y_ref * 0, a_ref)["ok"]
