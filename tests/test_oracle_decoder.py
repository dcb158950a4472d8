"""Pins of the oracle's small decoder and of its speculative rounds.

The decoder layers are not on the pages; they are pinned by the mathematics
that defines them:
  * RMSNorm: unit mean square with unit gains, invariance to scaling x;
  * rotary embedding: each pair is rotated (norms kept), position 0 is the
    identity, and q.k after rotation depends only on the position difference;
  * SwiGLU against scipy's logistic function; bf16 rounding on ties.
The round is pinned by the blog's claim ("How Speculative Decoding Speeds Up
Inference", section "The same output as the large model alone"): with greedy
decoding, speculative rounds emit exactly the tokens of one target pass per
token. In the oracle every position is computed row by row and, in the exact
attention mode, sees the cache as a one-token pass would, so the claim holds
token for token and logit for logit; a bookkeeping mistake in a round (a
wrong position, a wrong number of committed tokens, the bonus taken from
the wrong row) breaks it.
"""
import numpy as np
import pytest
from scipy.special import expit

from nested_quantized_weights_amd import synth


@pytest.fixture(scope="module")
def D(oracle):
    from oracle import decoder

    return decoder


@pytest.fixture(scope="module")
def tiny(D):
    cfg = synth.TINY_DECODER
    return D.Decoder(cfg, synth.decoder_weights(cfg, (800,)))


def test_rmsnorm(D):
    x = synth.normal((6, 512), (810,))
    y = D.rmsnorm(x, np.ones(512, np.float32), 0.0)
    assert np.allclose(np.mean(y.astype(np.float64) ** 2, axis=1), 1.0, rtol=1e-6)
    assert np.array_equal(D.rmsnorm(4.0 * x, np.ones(512, np.float32), 0.0), y)  # exact power-of-two scale
    g = synth.normal(512, (811,))
    assert np.allclose(D.rmsnorm(x, g, 0.0), y * g, rtol=1e-6, atol=1e-7)


def test_rope(D):
    q = synth.normal((5, 3, 128), (812,)).astype(np.float64)
    k = synth.normal((5, 3, 128), (813,)).astype(np.float64)
    pos = np.array([0, 1, 7, 100, 1000])
    rq = D.rope(q, pos, 10000.0)
    assert np.array_equal(rq[0], q[0])  # position 0: identity
    n0 = q[..., :64] ** 2 + q[..., 64:] ** 2
    n1 = rq[..., :64] ** 2 + rq[..., 64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)  # a rotation per pair
    for shift in (3, 250):
        a = np.sum(D.rope(q, pos, 1e4) * D.rope(k, pos[::-1], 1e4), axis=-1)
        b = np.sum(D.rope(q, pos + shift, 1e4) * D.rope(k, pos[::-1] + shift, 1e4), axis=-1)
        assert np.allclose(a, b, rtol=1e-9, atol=1e-9)  # depends on the position difference only


def test_swiglu_and_bf16(D):
    gu = synth.normal((3, 200), (814,))
    g, u = gu[:, :100].astype(np.float64), gu[:, 100:].astype(np.float64)
    assert np.allclose(D.swiglu(gu), g * expit(g) * u, rtol=1e-6, atol=1e-7)
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0], np.float32)
    assert list(D.bf16_bits(v)) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000]


@pytest.mark.parametrize("k", [1, 3, 4])
def test_speculative_rounds_emit_the_target_only_tokens(tiny, k):
    prompt = synth.tokens(40, tiny.cfg["vocab"], (801,))
    ar, r_ar = tiny.generate(prompt, 48, 0)
    sp, r_sp = tiny.generate(prompt, 48, k, exact=True)
    assert sp == ar
    # logit for logit: position j's target logits are the same in both runs
    y_ar = np.concatenate([y for _, y in r_ar])
    y_sp = np.concatenate([y for _, y in r_sp])[:len(y_ar)]
    assert np.array_equal(y_sp.view(np.uint32), y_ar[:len(y_sp)].view(np.uint32))
    # the rounds did speculate: more than one token per target pass
    assert np.mean([n for n, _ in r_sp]) > 1.5


def test_round_bookkeeping_mistakes_break_the_claim(tiny, D):
    # a round that commits one token too many (the first rejected draft
    # kept) emits a different sequence: the claim test has power
    prompt = synth.tokens(40, tiny.cfg["vocab"], (801,))
    ar, _ = tiny.generate(prompt, 48, 0)

    class Greedy(D.Decoder):
        def generate(self, prompt, n_new, k, exact=True):
            from oracle import oracle as O

            self.reset()
            t, pos = self.prefill(prompt)
            out = []
            while len(out) < n_new:
                drafts, x = [], t
                for j in range(k):
                    x = O.argmax(self.logits(self.forward([x], pos + j, draft=True), draft=True)[0])
                    drafts.append(x)
                y = self.logits(self.forward([t] + drafts, pos, draft=False), draft=False)
                a = 0
                while a < k and drafts[a] == O.argmax(y[a]):
                    a += 1
                a = min(a + 1, k)  # planted mistake
                emitted = drafts[:a] + [O.argmax(y[a])]
                out += emitted
                pos += len(emitted)
                t = emitted[-1]
            return out[:n_new], []

    bad = Greedy.__new__(Greedy)
    bad.__dict__.update(tiny.__dict__)
    sp, _ = bad.generate(prompt, 48, 4)
    assert sp != ar


def test_teacher_forced_logits_are_those_of_target_only_decoding(tiny):
    # scoring a sequence position by position from its own prefix (16
    # positions per exact target pass) must give, bit for bit, the logits
    # that target-only decoding computed when it produced that sequence: an
    # off-by-one in the start row or in the positions would shift them
    prompt = synth.tokens(40, tiny.cfg["vocab"], (801,))
    ar, r_ar = tiny.generate(prompt, 20, 0)
    y_ar = np.concatenate([y for _, y in r_ar])[:len(ar)]
    y_tf = tiny.teacher_forced_logits(list(prompt) + list(ar), len(prompt) - 1)
    assert y_tf.shape == y_ar.shape
    assert np.array_equal(y_tf.view(np.uint32), y_ar.view(np.uint32))


def test_attention_noise_has_its_stated_relative_norm(D):
    # the noise the decoder-vs-oracle tolerance is derived from: every
    # attention output vector (per position and head) moves by exactly
    # att_noise times its norm, the same seed gives the same draw, and
    # att_noise = 0 leaves the computation untouched
    cfg = synth.TINY_DECODER
    w = synth.decoder_weights(cfg, (800,))
    d, Hq = cfg["head_dim"], cfg["q_heads"]

    class Capture(D.Decoder):
        def linear(self, x, packed, draft):
            if any(packed is lw["o"] for lw in self.layers):
                self.seen.append(np.array(x, np.float64).reshape(len(x), Hq, d))
            return D.Decoder.linear(x, packed, draft)

    toks = synth.tokens(12, cfg["vocab"], (802,))
    outs = {}
    for key, noise, seed in (("plain", 0.0, 0), ("zero", 0.0, 5), ("a", 2e-3, 1), ("b", 2e-3, 1)):
        dec = Capture(cfg, w, att_noise=noise, noise_seed=seed)
        dec.seen = []
        h = dec.forward(list(toks), 0, draft=False, exact=True)
        outs[key] = (dec.seen, h)
    assert np.array_equal(outs["plain"][1], outs["zero"][1])
    assert np.array_equal(outs["a"][1], outs["b"][1])
    assert not np.array_equal(outs["a"][1], outs["plain"][1])
    # first layer: same inputs, so the attention outputs differ by the noise alone
    att0, att1 = outs["plain"][0][0], outs["a"][0][0]
    rel = np.linalg.norm(att1 - att0, axis=-1) / np.linalg.norm(att0, axis=-1)
    assert np.allclose(rel, 2e-3, rtol=1e-3), (rel.min(), rel.max())
