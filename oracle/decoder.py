"""Plain CPU reference of a small pre-norm decoder run through speculative
rounds end to end.

TEST INFRASTRUCTURE ONLY: the checker, not the product. Only the tests, the
package's smoke check and the CPU-baseline leg of the benchmark may use it.
It imports nothing from the HIP library.

The decoder layers are not on the pages; they are the plain Llama/Qwen-style
ones (RMSNorm, rotate-half rotary embedding, grouped-query attention, SwiGLU),
written here in fp64 and stored in fp32 between steps. The nested parts are
the oracle's own: per-token int8 activations, the W4A8 draft and W8A8
target linears (BitNest, Figure 3), and the nested KV cache with its
append and the base / full views (BitNest, Figure 4). The round is the
blog's ("How Speculative Decoding Speeds Up Inference", Table 1 and the
section "The same output as the large model alone"): the draft proposes k
tokens, one target pass scores k+1 positions, drafts are kept while they
equal the target's top choice, and the target's choice at the first
mismatch (or the bonus) is emitted.

Two ways to attend in a target pass over k+1 positions:
  exact    position by position: append one token's K/V, attend with its
           query, then the next; each query sees the cache exactly as a
           one-token-per-pass decode would;
  batched  append all k+1 tokens, then attend with all k+1 queries; an open
           128-token block is then quantized with the later positions of the
           pass included, so earlier queries see slightly different K/V.
Every position is computed row by row, so a position's result does not
depend on how many positions share its pass.
"""
from __future__ import annotations

import numpy as np

from . import oracle as O


def rmsnorm(x, gamma, eps):
    """x / sqrt(mean(x^2) + eps) * gamma per row, in fp64, stored fp32."""
    x = np.asarray(x, np.float64)
    out = np.empty(x.shape, np.float32)
    for m in range(x.shape[0]):
        r = 1.0 / np.sqrt(np.mean(x[m] * x[m]) + eps)
        out[m] = (x[m] * r * np.asarray(gamma, np.float64)).astype(np.float32)
    return out


def rope(x, positions, theta):
    """Rotate-half rotary embedding of x [M][heads][d] at positions [M]:
    pair (i, i + d/2) turned by pos * theta^(-2i/d). fp64 in, fp64 out."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half) / d)
    out = np.empty_like(x)
    for m, p in enumerate(positions):
        ang = p * inv
        c, s = np.cos(ang), np.sin(ang)
        x1, x2 = x[m, :, :half], x[m, :, half:]
        out[m, :, :half] = x1 * c - x2 * s
        out[m, :, half:] = x2 * c + x1 * s
    return out


def swiglu(gate_up):
    """silu(g) * u for gate_up [M][2I] = [g | u], in fp64, stored fp32."""
    gu = np.asarray(gate_up, np.float64)
    I = gu.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    return (g / (1.0 + np.exp(-g)) * u).astype(np.float32)


def bf16_bits(x):
    """fp32 -> bf16 bit patterns, nearest with ties to even."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


class Decoder:
    """The decoder with nested weights and one nested KV cache per layer."""

    def __init__(self, cfg, weights, att_noise=0.0, noise_seed=0):
        """att_noise > 0 adds to every attention output vector (per position
        and head) a random vector of att_noise times its norm: a test of how
        far the logits move when attention is off by a given normwise
        tolerance. 0 (the default) leaves the computation untouched."""
        self.cfg = cfg
        self.att_noise = float(att_noise)
        self.noise_rng = np.random.default_rng(noise_seed)
        self.embed = np.asarray(weights["embed"], np.float32)
        self.norm_final = weights["norm_final"]
        self.head = O.nest_pack(weights["lm_head"])
        self.layers = []
        for lw in weights["layers"]:
            self.layers.append({"norm_attn": lw["norm_attn"], "norm_mlp": lw["norm_mlp"],
                                **{n: O.nest_pack(lw[n]) for n in ("qkv", "o", "gate_up", "down")}})
        self.reset()

    def reset(self):
        c = self.cfg
        shape = (c["kv_heads"], c["capacity"], c["head_dim"])
        self.kv = []
        for _ in self.layers:
            kf, vf = np.zeros(shape, np.float32), np.zeros(shape, np.float32)
            self.kv.append((O.kv_nest_pack(kf, vf), kf, vf))

    @staticmethod
    def linear(x, packed, draft):
        """Per-token int8 activations, then the draft (base plane) or target
        (both planes) linear."""
        base, refine, scales = packed
        qa, sa = O.act_quant(x)
        return O.draft_gemv(qa, sa, base, scales) if draft else O.verify_gemm(qa, sa, base, refine, scales)

    def forward(self, tokens, pos0, draft, exact=True):
        """Hidden states after the final norm for tokens at pos0.., and the
        cache updated with their K/V. draft: base planes and the base KV
        view; else both planes and the full view."""
        c = self.cfg
        M = len(tokens)
        Hq, Hkv, d = c["q_heads"], c["kv_heads"], c["head_dim"]
        view = 0 if draft else 1
        positions = np.arange(pos0, pos0 + M)
        x = self.embed[np.asarray(tokens)].astype(np.float32)
        for lw, (kv, kf, vf) in zip(self.layers, self.kv):
            h = rmsnorm(x, lw["norm_attn"], c["eps"])
            qkv = self.linear(h, lw["qkv"], draft).reshape(M, Hq + 2 * Hkv, d)
            q = bf16_bits(rope(qkv[:, :Hq], positions, c["theta"]).astype(np.float32))
            k = rope(qkv[:, Hq:Hq + Hkv], positions, c["theta"]).astype(np.float32)
            v = qkv[:, Hq + Hkv:].astype(np.float32)
            k_new = np.ascontiguousarray(k.transpose(1, 0, 2))  # [Hkv][M][d]
            v_new = np.ascontiguousarray(v.transpose(1, 0, 2))
            if exact:
                att = np.empty((M, Hq, d), np.float32)
                for i in range(M):
                    O.kv_append(kv, kf, vf, k_new[:, i:i + 1], v_new[:, i:i + 1], pos0 + i)
                    att[i] = O.kv_attend(q[i:i + 1], kv, pos0 + i + 1, view)[0]
            else:
                O.kv_append(kv, kf, vf, k_new, v_new, pos0)
                att = O.kv_attend(q, kv, pos0 + M, view).astype(np.float32)
            if self.att_noise > 0.0:
                u = self.noise_rng.standard_normal(att.shape)
                u *= (self.att_noise * np.linalg.norm(att, axis=-1, keepdims=True)
                      / np.linalg.norm(u, axis=-1, keepdims=True))
                att = (att + u).astype(np.float32)
            x = (x + self.linear(att.reshape(M, Hq * d), lw["o"], draft)).astype(np.float32)
            h = rmsnorm(x, lw["norm_mlp"], c["eps"])
            x = (x + self.linear(swiglu(self.linear(h, lw["gate_up"], draft)), lw["down"], draft)).astype(np.float32)
        return rmsnorm(x, self.norm_final, c["eps"])

    def logits(self, h, draft):
        return self.linear(h, self.head, draft)

    def prefill(self, prompt):
        """Target passes over prompt[:-1] (16 positions at a time, exact
        attention); returns the round input (last prompt token, its position)."""
        n = len(prompt) - 1
        for s in range(0, n, 16):
            self.forward(prompt[s:min(n, s + 16)], s, draft=False, exact=True)
        return int(prompt[-1]), n

    def teacher_forced_logits(self, tokens, start):
        """Target logits of every position from start on, each computed from
        the sequence's own prefix: one exact target pass over tokens[:-1],
        16 positions at a time, so row j holds what target-only decoding
        would score after tokens[start + j]. [len(tokens) - 1 - start][V]."""
        self.reset()
        n = len(tokens) - 1
        rows = []
        for s in range(0, n, 16):
            h = self.forward(list(tokens[s:min(n, s + 16)]), s, draft=False, exact=True)
            if s + h.shape[0] > start:
                y = self.logits(h, draft=False)
                rows.append(y[max(0, start - s):])
        return np.concatenate(rows)

    def generate(self, prompt, n_new, k, exact=True):
        """Greedy decoding of n_new tokens after the prompt. k = 0: one target
        pass per token. k > 0: speculative rounds of k draft steps and one
        target pass. Returns (tokens, rounds) with rounds a list of
        (emitted count, logits of the emitted positions [n][V])."""
        self.reset()
        t, pos = self.prefill(prompt)
        out, rounds = [], []
        while len(out) < n_new:
            drafts = []
            x = t
            for j in range(k):
                h = self.forward([x], pos + j, draft=True, exact=True)
                x = O.argmax(self.logits(h, draft=True)[0])
                drafts.append(x)
            h = self.forward([t] + drafts, pos, draft=False, exact=exact)
            y = self.logits(h, draft=False)
            tgt = [O.argmax(y[i]) for i in range(k + 1)]
            a = 0
            while a < k and drafts[a] == tgt[a]:
                a += 1
            emitted = drafts[:a] + [tgt[a]]
            rounds.append((a + 1, y[:a + 1]))
            out += emitted
            pos += a + 1
            t = emitted[-1]
        return out[:n_new], rounds
