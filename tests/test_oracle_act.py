"""Pins of the oracle's per-token int8 activation quantizer (CPU only).

What fixes the expected values: a hand-derived example
(tests/golden/act_hand_example.json: ties to even, the zero row) and the
closed forms |x - sa*qa| <= sa/2, the max-abs element maps to +-127, and
sa = max|x|/127 in fp32.
"""
import json
import os

import numpy as np

from nested_quantized_weights_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_example(oracle):
    ex = json.load(open(os.path.join(GOLDEN, "act_hand_example.json")))
    qa, sa = oracle.act_quant(np.array(ex["x"], np.float32))
    assert sa.tolist() == ex["sa"]
    assert qa.tolist() == ex["qa"]


def test_closed_forms(oracle):
    x = synth.activations(17, 3584, (95,))
    x[3] *= 1e-3
    x[5] *= 1e3
    qa, sa = oracle.act_quant(x)
    assert np.array_equal(sa, (np.abs(x).max(axis=1) / np.float32(127)).astype(np.float32))
    assert qa.min() >= -127
    err = np.abs(x.astype(np.float64) - sa[:, None].astype(np.float64) * qa)
    assert np.all(err <= sa[:, None] * (0.5 + 1e-6))
    i = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(qa[np.arange(17), i]) == 127)
    assert np.all(np.sign(qa[np.arange(17), i]) == np.sign(x[np.arange(17), i]))
