"""A small pre-norm decoder run through greedy speculative rounds on the GPU.

Every computation is a call into the HIP library (nestspec): nest_embed,
nest_add_rmsnorm, nest_rope_split and nest_swiglu for the layers around the
nested linears (draft_gemv_x over the base planes, verify_gemm_x over both),
kv_nest_append / kv_nest_attend on one nested KV cache per layer (base view
for the draft, full view for the target), and draft_gemv_x / verify_accept_x
with the fused argmax on the nested LM head. This module only sequences the
calls and keeps positions (the round of "How Speculative Decoding Speeds Up
Inference", Table 1).

A target pass over the k+1 positions of a round attends either
  exact    position by position (append one token, attend with its query),
           so each query sees the cache a one-token pass would see; with
           row-independent layers the round then emits exactly the tokens
           and logits of target-only decoding ("The same output as the
           large model alone"), or
  batched  with one append of all k+1 tokens and one attention of all k+1
           queries (what the benchmark's round does), where the open block
           is quantized with the later positions of the pass included.
"""
from __future__ import annotations

import numpy as np
import torch

from . import nestspec as ns


class Decoder:
    def __init__(self, cfg: dict, weights: dict, device: str = "cuda"):
        self.cfg = cfg
        self.dev = torch.device(device)

        def t(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

        self.embed = t(weights["embed"])
        self.norm_final = t(weights["norm_final"])
        self.head = ns.nest_pack_tiled(t(weights["lm_head"]))
        self.layers = []
        for lw in weights["layers"]:
            self.layers.append({"norm_attn": t(lw["norm_attn"]), "norm_mlp": t(lw["norm_mlp"]),
                                **{n: ns.nest_pack_tiled(t(lw[n])) for n in ("qkv", "o", "gate_up", "down")}})
        self.no_draft = torch.zeros(1, dtype=torch.int32, device=self.dev)
        self.reset()

    def reset(self):
        c = self.cfg
        shape = (c["kv_heads"], c["capacity"], c["head_dim"])
        z = torch.zeros(shape, dtype=torch.float32, device=self.dev)
        self.kv = []
        for _ in self.layers:
            kv = ns.kv_nest_pack(z, z)
            sh = ns.kv_shadow(kv)
            ns.kv_nest_shadow_fill(kv, z, z, 0, sh)
            self.kv.append((kv, sh))

    def _linear(self, x, W, draft):
        return ns.draft_gemv_x(x, W) if draft else ns.verify_gemm_x(x, W)

    def forward(self, tokens: torch.Tensor, pos0: int, draft: bool, exact: bool = True) -> torch.Tensor:
        """Hidden states after the final norm for int32 tokens [M] at
        positions pos0.., with their K/V appended to every layer's cache."""
        c = self.cfg
        M = tokens.numel()
        Hq, Hkv, d, eps = c["q_heads"], c["kv_heads"], c["head_dim"], c["eps"]
        view = 0 if draft else 1
        x = ns.embed(self.embed, tokens)
        h = torch.empty_like(x)
        dn = None
        for lw, (kv, sh) in zip(self.layers, self.kv):
            ns.add_rmsnorm(x, dn, lw["norm_attn"], eps, out=h)
            qkv = self._linear(h, lw["qkv"], draft)
            q, k, v = ns.rope_split(qkv, pos0, Hq, Hkv, d, c["theta"], token_major=exact)
            if exact:
                att = torch.empty((M, Hq, d), dtype=torch.float32, device=self.dev)
                for i in range(M):
                    ns.kv_nest_append(kv, sh, k[i].unsqueeze(1), v[i].unsqueeze(1), pos0 + i)
                    ns.kv_nest_attend(q[i:i + 1], kv, pos0 + i + 1, view, out=att[i:i + 1])
            else:
                ns.kv_nest_append(kv, sh, k, v, pos0)
                att = ns.kv_nest_attend(q, kv, pos0 + M, view)
            o = self._linear(att.view(M, Hq * d), lw["o"], draft)
            ns.add_rmsnorm(x, o, lw["norm_mlp"], eps, out=h)
            dn = self._linear(ns.swiglu(self._linear(h, lw["gate_up"], draft)), lw["down"], draft)
        ns.add_rmsnorm(x, dn, self.norm_final, eps, out=h)
        return h

    def prefill(self, prompt) -> tuple:
        """Target passes over prompt[:-1], 16 positions at a time with
        position-by-position attention; returns the round input (the last
        prompt token on the device, its position)."""
        p = torch.from_numpy(np.ascontiguousarray(prompt, np.int32)).to(self.dev)
        n = p.numel() - 1
        for s in range(0, n, 16):
            self.forward(p[s:min(n, s + 16)], s, draft=False, exact=True)
        return p[n:n + 1].clone(), n

    def generate(self, prompt, n_new: int, k: int, exact: bool = True):
        """Greedy decoding of n_new tokens after the prompt: one target pass
        per token when k = 0, else rounds of k draft steps and one target
        pass. Returns (tokens, rounds): rounds lists (emitted count, target
        logits of the emitted positions [n][V] on the device)."""
        self.reset()
        t, pos = self.prefill(prompt)
        out, rounds = [], []
        while len(out) < n_new:
            toks = torch.empty(k + 1, dtype=torch.int32, device=self.dev)
            toks[0:1] = t
            for j in range(k):
                h = self.forward(toks[j:j + 1], pos + j, draft=True, exact=True)
                ns.draft_gemv_x(h, self.head, want_y=False, argmax=True, argmax_out=toks[j + 1:j + 2])
            h = self.forward(toks, pos, draft=False, exact=exact)
            res = ns.verify_accept_x(h, 1, k, self.head, toks[1:] if k else self.no_draft, want_y=True)
            n = int(res["n_emitted"][0].item())
            out += res["emitted"][0, :n].tolist()
            rounds.append((n, res["y"][:n]))
            pos += n
            t = res["emitted"][0, n - 1:n].clone()
        return out[:n_new], rounds
