"""Pins of the oracle's draft and verify products (CPU only).

What fixes the expected values:
  * brute force: an int64 numpy matmul, per group, of codes decoded
    independently from the planes (tests/formats.py), on tiny shapes with
    N != K (a transposed operand fails) and ragged M;
  * the exact value: an fp64 fold of the same exact group sums. The fp32
    result must fall within the rounding bound (G+2) * 2^-24 * A with
    A = sa * sum_g |s_g * A_g|. A dropped term, a wrong scale (s instead of
    s/16) or a missing activation scale fails this by orders of magnitude;
  * BitNest, Figure 3: the draft's base-plane sums are the base part of
    the verify sums (Av = 16*Ab + Ar). With the refinement plane zeroed,
    verify equals draft bit for bit;
  * batch invariance: a row's outputs do not depend on the other rows.
"""
import numpy as np
import pytest

from formats import decode_matrix
from nested_quantized_weights_amd import synth

U32 = 2.0 ** -24


def _setup(N, K, M, key):
    w = synth.weights(N, K, (80,) + key)
    x = synth.activations(M, K, (81,) + key)
    return w, x


def _group_sums(qa, codes, group):
    M, K = qa.shape
    N = codes.shape[0]
    G = K // group
    a = qa.astype(np.int64).reshape(M, G, group)
    c = codes.astype(np.int64).reshape(N, G, group)
    return np.einsum("mgk,ngk->mng", a, c)


def _bound_check(y, sa, scales, acc, step):
    s = scales.astype(np.float64) * step  # [N][G]
    terms = s[None, :, :] * acc.astype(np.float64)  # [M][N][G]
    exact = sa.astype(np.float64)[:, None] * terms.sum(axis=2)
    A = sa.astype(np.float64)[:, None] * np.abs(terms).sum(axis=2)
    G = scales.shape[1]
    err = np.abs(y.astype(np.float64) - exact)
    assert np.all(err <= (G + 2) * U32 * A + 1e-45), float((err / (A + 1e-300)).max())


SHAPES = [(N, K, M) for N in (1, 3, 8, 33) for K in (128, 256, 384) for M in (1, 5, 9, 17)]


@pytest.mark.parametrize("N,K,M", SHAPES)
def test_brute_force(oracle, N, K, M):
    w, x = _setup(N, K, M, (N, K, M))
    base, refine, scales = oracle.nest_pack(w)
    qa, sa = oracle.act_quant(x)
    qb = decode_matrix(base, N, K)
    qr = decode_matrix(refine, N, K)

    yd, accd = oracle.draft_gemv(qa, sa, base, scales, want_acc=True)
    ab = _group_sums(qa, qb, 128)
    assert np.array_equal(accd, ab)
    _bound_check(yd, sa, scales, accd, 1.0)

    yv, accv = oracle.verify_gemm(qa, sa, base, refine, scales, want_acc=True)
    av = _group_sums(qa, 16 * qb.astype(np.int16) + qr, 128)
    assert np.array_equal(accv, av)
    assert np.array_equal(accv, 16 * ab + _group_sums(qa, qr, 128))
    _bound_check(yv, sa, scales, accv, 1.0 / 16)


def test_zero_refinement_makes_verify_equal_draft(oracle):
    w, x = _setup(40, 512, 9, (7,))
    base, refine, scales = oracle.nest_pack(w)
    qa, sa = oracle.act_quant(x)
    yd = oracle.draft_gemv(qa, sa, base, scales)
    yv = oracle.verify_gemm(qa, sa, base, np.zeros_like(refine), scales)
    assert np.array_equal(yd.view(np.uint32), yv.view(np.uint32))


def test_batch_invariance(oracle):
    w, x = _setup(24, 768, 9, (8,))
    base, refine, scales = oracle.nest_pack(w)
    qa, sa = oracle.act_quant(x)
    y9 = oracle.verify_gemm(qa, sa, base, refine, scales)
    for m in (0, 4, 8):
        y1 = oracle.verify_gemm(qa[m:m + 1], sa[m:m + 1], base, refine, scales)
        assert np.array_equal(y1[0].view(np.uint32), y9[m].view(np.uint32))


def test_tracks_float_matmul(oracle):
    # Sanity on meaning: the verify product approximates x @ W^T to within
    # the 8-bit weight and 8-bit activation quantization error.
    w, x = _setup(64, 1024, 4, (9,))
    base, refine, scales = oracle.nest_pack(w)
    qa, sa = oracle.act_quant(x)
    yv = oracle.verify_gemm(qa, sa, base, refine, scales).astype(np.float64)
    yd = oracle.draft_gemv(qa, sa, base, scales).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    rel_v = np.linalg.norm(yv - ref) / np.linalg.norm(ref)
    rel_d = np.linalg.norm(yd - ref) / np.linalg.norm(ref)
    assert rel_v < 0.03
    assert rel_v < rel_d < 0.3  # the refinement recovers precision


def test_argmax_lowest_index_among_ties(oracle):
    y = np.array([1.0, 3.0, -2.0, 3.0, 3.0], np.float32)
    assert oracle.argmax(y) == 1 == int(np.argmax(y))
    z = np.array([-0.0, 0.0, -0.0], np.float32)
    assert oracle.argmax(z) == 0
    g = synth.rng(83)
    for _ in range(50):
        v = g.integers(-3, 4, size=int(g.integers(1, 40))).astype(np.float32)
        assert oracle.argmax(v) == int(np.argmax(v))
