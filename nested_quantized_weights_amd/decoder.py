"""A small pre-norm decoder run through greedy speculative rounds on the GPU.

Every computation is a call into the HIP library (nestspec): nest_embed,
nest_add_rmsnorm, nest_rope_split and nest_swiglu for the layers around the
nested linears (draft_gemv_x over the base planes, verify_gemm_x over both),
kv_nest_append / kv_nest_attend (one position) and
kv_nest_append_attend_exact (a verify pass) on one nested KV cache per layer
(base view for the draft, full view for the target), and draft_gemv_x /
verify_accept_x with the fused argmax on the nested LM head. This module only sequences the
calls (the round of "How Speculative Decoding Speeds Up Inference", Table 1).

Round state lives on the device: the committed cache length (one int32,
advanced by verify_accept by the tokens it emits) and each round's token
buffer, whose slot 0 verify_accept fills with the next round's input. Every
position and context length is that device length plus a host offset, so
rounds can be issued back to back without the host reading anything
(run_rounds); generate() reads each round's count only to know when to stop.

A target pass over the k+1 positions of a round attends in one of three ways:
  exact     kv_nest_append_attend_exact: the append of the k+1 tokens and
            one attention launch in which each query sees the cache a
            one-token pass at its position would see (its open block
            quantized over its own prefix); with row-independent layers the
            round then emits exactly the tokens and logits of target-only
            decoding ("The same output as the large model alone");
  stepwise  position by position (append one token, attend with its
            query): the same result with k+1 launches of each;
  batched   one append and one attention of all k+1 queries, where the open
            block is quantized with the later positions of the pass included.
"""
from __future__ import annotations

import time

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
        self.length = torch.zeros(1, dtype=torch.int32, device=self.dev)  # committed cache length
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
        self.length.zero_()

    def _linear(self, x, W, draft):
        return ns.draft_gemv_x(x, W) if draft else ns.verify_gemm_x(x, W)

    def forward(self, tokens: torch.Tensor, off: int, draft: bool, mode: str = "exact") -> torch.Tensor:
        """Hidden states after the final norm for int32 tokens [M] at
        positions length + off.. (length on the device), with their K/V
        appended to every layer's cache; mode is how a multi-token pass
        attends (module docstring)."""
        if mode not in ("exact", "stepwise", "batched"):
            raise ValueError(f"mode {mode!r}")
        c = self.cfg
        M = tokens.numel()
        Hq, Hkv, d, eps = c["q_heads"], c["kv_heads"], c["head_dim"], c["eps"]
        view = 0 if draft else 1
        L = self.length
        x = ns.embed(self.embed, tokens)
        h = torch.empty_like(x)
        dn = None
        for lw, (kv, sh) in zip(self.layers, self.kv):
            ns.add_rmsnorm(x, dn, lw["norm_attn"], eps, out=h)
            qkv = self._linear(h, lw["qkv"], draft)
            stepwise = mode == "stepwise"
            q, k, v = ns.rope_split(qkv, off, Hq, Hkv, d, c["theta"], token_major=stepwise, pos_dev=L)
            if stepwise:
                att = torch.empty((M, Hq, d), dtype=torch.float32, device=self.dev)
                for i in range(M):
                    ns.kv_nest_append(kv, sh, k[i].unsqueeze(1), v[i].unsqueeze(1), off + i, pos_dev=L)
                    ns.kv_nest_attend(q[i:i + 1], kv, off + i + 1, view, out=att[i:i + 1], ctx_dev=L)
            elif mode == "exact" and M > 1:
                # the append and the exact attention in one call
                att = ns.kv_nest_append_attend_exact(q, kv, sh, k, v, off, view, pos_dev=L)
            else:
                ns.kv_nest_append(kv, sh, k, v, off, pos_dev=L)
                # one position: the append quantized its block over exactly
                # the tokens up to it, so every mode is the plain attention
                att = ns.kv_nest_attend(q, kv, off + M, view, ctx_dev=L)
            o = self._linear(att.view(M, Hq * d), lw["o"], draft)
            ns.add_rmsnorm(x, o, lw["norm_mlp"], eps, out=h)
            dn = self._linear(ns.swiglu(self._linear(h, lw["gate_up"], draft)), lw["down"], draft)
        ns.add_rmsnorm(x, dn, self.norm_final, eps, out=h)
        return h

    def prefill(self, prompt) -> torch.Tensor:
        """Target passes over prompt[:-1], 16 positions at a time with
        position-by-position attention; leaves the committed length at
        len(prompt) - 1 and returns the last prompt token on the device."""
        self.reset()
        p = torch.from_numpy(np.ascontiguousarray(prompt, np.int32)).to(self.dev)
        n = p.numel() - 1
        for s in range(0, n, 16):
            self.forward(p[s:min(n, s + 16)], s, draft=False, mode="exact")
        self.length.fill_(n)
        return p[n:n + 1]

    def _buffers(self, rounds: int, k: int, want_y: bool):
        V = self.head.rows
        E = torch.empty
        return {"toks": E((rounds + 1, k + 1), dtype=torch.int32, device=self.dev),
                "target": E((rounds, k + 1), dtype=torch.int32, device=self.dev),
                "n_emitted": E((rounds, 1), dtype=torch.int32, device=self.dev),
                "emitted": E((rounds, k + 1), dtype=torch.int32, device=self.dev),
                "y": E((rounds, k + 1, V), dtype=torch.float32, device=self.dev) if want_y else None}

    def _round(self, r: int, k: int, mode: str, b: dict):
        """Issue round r: k draft steps and one target pass. Slot 0 of
        b["toks"][r] holds the round's input; verify_accept advances the
        committed length and writes the next round's input."""
        toks = b["toks"][r]
        for j in range(k):
            h = self.forward(toks[j:j + 1], j, draft=True, mode="exact")
            ns.draft_gemv_x(h, self.head, want_y=False, argmax=True, argmax_out=toks[j + 1:j + 2])
        h = self.forward(toks, 0, draft=False, mode=mode)
        out = {"target": b["target"][r], "n_emitted": b["n_emitted"][r], "emitted": b["emitted"][r]}
        if b["y"] is not None:
            out["y"] = b["y"][r]
        ns.verify_accept_x(h, 1, k, self.head, toks[1:] if k else self.no_draft, out=out,
                           length=self.length, next_token=b["toks"][r + 1][0:1])

    def run_rounds(self, prompt, rounds: int, k: int, mode: str = "exact", want_y: bool = True, timing=None):
        """A fixed number of rounds issued back to back with no host read
        between them (positions, lengths and inputs advance on the device).
        Returns (tokens, per round (emitted count, logits of the emitted
        positions [n][V] or None)) after one synchronisation at the end;
        timing, a dict, receives the rounds' wall-clock seconds."""
        b = self._buffers(rounds, k, want_y)
        b["toks"][0, 0:1].copy_(self.prefill(prompt))
        torch.cuda.synchronize(self.dev)
        t0 = time.perf_counter()
        for r in range(rounds):
            self._round(r, k, mode, b)
        torch.cuda.synchronize(self.dev)
        if timing is not None:
            timing["rounds_s"] = time.perf_counter() - t0
        n = b["n_emitted"][:, 0].cpu().numpy()
        em = b["emitted"].cpu().numpy()
        toks, per = [], []
        for r in range(rounds):
            toks += em[r, :n[r]].tolist()
            per.append((int(n[r]), b["y"][r, :n[r]] if want_y else None))
        return toks, per

    def graph_rounds(self, prompt, rounds: int, k: int, mode: str = "exact", sync_each: bool = False,
                     timing=None):
        """The same rounds as run_rounds, with round 0 issued eagerly and every
        later round a replay of one HIP graph of a round (captured after
        round 0, on a stream of its own). A round reads its input token from
        and writes the next one to one device buffer, and appends its emitted
        tokens and count to a device ring at a device-held index, so a replay
        needs no host work at all. sync_each synchronizes after every replay
        and reads the ring index (eager work between replays); timing, a
        dict, receives the replays' wall-clock seconds. Returns (tokens,
        emitted counts)."""
        dev = self.dev
        k1 = k + 1
        toks = torch.empty(k1, dtype=torch.int32, device=dev)  # [0]: the round's input
        out = {"target": torch.empty(k1, dtype=torch.int32, device=dev),
               "n_emitted": torch.empty(1, dtype=torch.int32, device=dev),
               "emitted": torch.empty(k1, dtype=torch.int32, device=dev)}
        ring_t = torch.full((rounds, k1), -1, dtype=torch.int32, device=dev)
        ring_n = torch.zeros(rounds, dtype=torch.int32, device=dev)
        ring_i = torch.zeros(1, dtype=torch.int64, device=dev)

        def one_round():
            for j in range(k):
                h = self.forward(toks[j:j + 1], j, draft=True, mode="exact")
                ns.draft_gemv_x(h, self.head, want_y=False, argmax=True, argmax_out=toks[j + 1:j + 2])
            h = self.forward(toks, 0, draft=False, mode=mode)
            ns.verify_accept_x(h, 1, k, self.head, toks[1:] if k else self.no_draft, out=dict(out),
                               length=self.length, next_token=toks[0:1])
            ring_t.index_copy_(0, ring_i, out["emitted"].view(1, k1))
            ring_n.index_copy_(0, ring_i, out["n_emitted"])
            ring_i.add_(1)

        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            toks[0:1].copy_(self.prefill(prompt))
            one_round()  # round 0, eager: also sets up every workspace on this stream
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                one_round()
            side.synchronize()
            t0 = time.perf_counter()
            for r in range(rounds - 1):
                graph.replay()
                if sync_each:
                    side.synchronize()
                    if int(ring_i.item()) != r + 2:
                        raise RuntimeError(f"replay {r}: ring index {int(ring_i.item())}")
            side.synchronize()
            if timing is not None:
                timing["replay_s"] = time.perf_counter() - t0
        torch.cuda.current_stream(dev).wait_stream(side)
        n = ring_n.cpu().numpy()
        t = ring_t.cpu().numpy()
        tokens = []
        for r in range(rounds):
            tokens += t[r, :n[r]].tolist()
        return tokens, n.tolist()

    def generate(self, prompt, n_new: int, k: int, mode: str = "exact"):
        """Greedy decoding of n_new tokens after the prompt: one target pass
        per token when k = 0, else rounds of k draft steps and one target
        pass; each round's emitted count is read back to know when to stop.
        Returns (tokens, rounds): rounds lists (emitted count, target logits
        of the emitted positions [n][V] on the device)."""
        b = self._buffers(n_new, k, True)
        b["toks"][0, 0:1].copy_(self.prefill(prompt))
        out, rounds, r = [], [], 0
        while len(out) < n_new:
            self._round(r, k, mode, b)
            n = int(b["n_emitted"][r, 0].item())
            out += b["emitted"][r, :n].tolist()
            rounds.append((n, b["y"][r, :n]))
            r += 1
        return out[:n_new], rounds
