"""The kernels' fast activation quantization rule, checked on the CPU.

The HIP kernels quantize x with t = x * r, r = 1/s_a (both IEEE fp32
products/quotients), and take the exact quotient x / s_a only when t lies
within 3e-5 of a half-integer. This test emulates that rule in numpy fp32
(IEEE round-to-nearest, as the GPU's v_mul_f32 / v_rcp-free division) and
checks it equals the oracle's plain rule clamp(rint(x / s_a), +-127) on
random rows, rows built on and around ties, tiny and huge scales, and -0.
"""
import numpy as np
import pytest

from nested_quantized_weights_amd import synth


def fast_rule(x, s):
    x = x.astype(np.float32)
    s = np.float32(s)
    if s == 0:
        return np.zeros(x.shape, np.int8)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        r = np.float32(1.0) / s
        t = (x * r).astype(np.float32)
        frac = (t - np.floor(t)).astype(np.float32)
        near = ~(np.abs((frac - np.float32(0.5)).astype(np.float32)) > np.float32(3e-5)) | ~(r < np.inf)
        q = np.where(near, np.rint((x / s).astype(np.float32)), np.rint(t))
    return np.clip(q, -127, 127).astype(np.int8)


def rows(seed):
    g = synth.rng(seed)
    out = [synth.activations(4, 4096, (seed, 0))]
    for mx in (1.0, 100.0, 127.0, 3e-30, 7e37, 0.3):
        s = np.float32(np.float32(mx) / np.float32(127.0))
        n = g.integers(-127, 127, size=4096).astype(np.float32)
        v = ((n + np.float32(0.5)) * s).astype(np.float32)
        for k in range(3):
            v = np.where(g.random(4096) < 0.3, np.nextafter(v, np.float32(np.inf)), v)
            v = np.where(g.random(4096) < 0.3, np.nextafter(v, np.float32(-np.inf)), v)
        v = np.clip(v, -np.float32(mx), np.float32(mx)).astype(np.float32)
        v[0] = np.float32(mx)
        v[1] = -0.0
        out.append(v[None])
    return np.concatenate(out).astype(np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fast_rule_equals_division_rule(oracle, seed):
    x = rows(400 + seed)
    qa, sa = oracle.act_quant(x)
    for m in range(x.shape[0]):
        assert np.array_equal(fast_rule(x[m], sa[m]), qa[m]), m
