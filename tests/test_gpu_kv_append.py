"""GPU parity of the KV write path (kv_nest_append, kv_nest_shadow_fill)
against the oracle's kv_append, bit-exact on every plane byte and scale.

A prefill packs the first ctx tokens (later tokens zero, so the open block's
scale covers its valid tokens), then rounds of speculative appends follow:
k+1 tokens at ctx, a random number kept (the caller's length update), the
next append writing over the rejected suffix. Positions cross block
boundaries, fill blocks exactly and start on a block boundary. The full-size
case appends to the 8-head 32K cache and attends over it.
"""
import numpy as np
import pytest
import torch

from nested_quantized_weights_amd import synth

pytestmark = pytest.mark.gpu
NAMES = ("k_base", "k_refine", "k_scale", "v_base", "v_refine", "v_scale")


@pytest.fixture(scope="module")
def ns():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nested_quantized_weights_amd import nestspec

    nestspec.lib()
    return nestspec


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same(kv, okv, heads=None):
    for n in NAMES:
        g, o = host(getattr(kv, n)), okv[n]
        if heads is not None:
            g = g.reshape(kv.n_kv_heads, -1)[heads]
            o = o.reshape(kv.n_kv_heads, -1)[heads]
        assert np.array_equal(g.view(np.uint8), o.view(np.uint8)), n


def prefill(ns, oracle, Hkv, cap, d, block, ctx, key):
    kf, vf = synth.kv(Hkv, cap, d, key)
    kf[:, ctx:] = 0.0
    vf[:, ctx:] = 0.0
    okv = oracle.kv_nest_pack(kf, vf, block=block)
    kd, vd = dev(kf), dev(vf)
    kv = ns.kv_nest_pack(kd, vd, block=block)
    sh = ns.kv_shadow(kv)
    ns.kv_nest_shadow_fill(kv, kd, vd, ctx, sh)
    return kv, sh, okv, kf, vf


@pytest.mark.parametrize("Hkv,d,block,ctx", [(2, 128, 128, 150), (2, 128, 128, 250), (1, 128, 128, 0),
                                             (3, 16, 32, 40), (2, 128, 128, 256)])
def test_append_rounds_bit_exact(ns, oracle, Hkv, d, block, ctx):
    cap = 6 * block
    kv, sh, okv, kf, vf = prefill(ns, oracle, Hkv, cap, d, block, ctx, (520, Hkv, d, block, ctx))
    same(kv, okv)
    g = synth.rng(521, Hkv, d, block, ctx)
    pos = ctx
    for rnd in range(12):
        k = int(g.integers(0, 9))
        if pos + k + 1 > cap:
            break
        nk, nv = synth.kv(Hkv, k + 1, d, (522, rnd, ctx))
        nk *= float(g.choice([1.0, 8.0]))  # some rounds dominate a scale
        ns.kv_nest_append(kv, sh, dev(nk), dev(nv), pos)
        oracle.kv_append(okv, kf, vf, nk, nv, pos)
        same(kv, okv)
        pos += int(g.integers(0, k + 1)) + 1  # a + 1 kept; the rest is overwritten next


def test_append_fills_block_exactly_then_seals(ns, oracle):
    Hkv, d, block, cap = 2, 128, 128, 3 * 128
    kv, sh, okv, kf, vf = prefill(ns, oracle, Hkv, cap, d, block, 119, (523,))
    nk, nv = synth.kv(Hkv, 9, d, (524,))
    ns.kv_nest_append(kv, sh, dev(nk), dev(nv), 119)  # exactly to the end of block 0
    oracle.kv_append(okv, kf, vf, nk, nv, 119)
    same(kv, okv)
    full = oracle.kv_nest_pack(kf, vf, block=block)  # block 0 is now the plain packed block
    assert np.array_equal(host(kv.k_scale)[:, 0], full["k_scale"][:, 0])
    nk2, nv2 = synth.kv(Hkv, block, d, (525,))
    ns.kv_nest_append(kv, sh, dev(nk2), dev(nv2), 128)  # a whole block in one call
    oracle.kv_append(okv, kf, vf, nk2, nv2, 128)
    same(kv, okv)


def test_full_size_append_then_attend(ns, oracle):
    wl = synth.WORKLOADS["kv_32k"]
    Hq, Hkv, d, ctx = wl["q_heads"], wl["kv_heads"], wl["head_dim"], wl["context"]
    cap, k = ctx + 128, 8
    kv, sh, okv, kf, vf = prefill(ns, oracle, Hkv, cap, d, 128, ctx, (526,))
    nk, nv = synth.kv(Hkv, k + 1, d, (527,))
    ns.kv_nest_append(kv, sh, dev(nk), dev(nv), ctx)
    oracle.kv_append(okv, kf, vf, nk, nv, ctx)
    same(kv, okv)
    q = synth.queries_bf16(k + 1, Hq, d, (528,))
    out = host(ns.kv_nest_attend(dev(q.view(np.int16)), kv, ctx + k + 1, 1))
    grp = Hq // Hkv
    for h in (0, 7):
        sub = {n: okv[n].reshape(Hkv, -1)[h:h + 1].reshape(-1) if n.endswith(("base", "refine"))
               else okv[n][h:h + 1] for n in NAMES}
        sub.update(n_kv_heads=1, capacity=cap, head_dim=d, block=128)
        ref = oracle.kv_attend(np.ascontiguousarray(q[:, h * grp:(h + 1) * grp]), sub, ctx + k + 1, 1)
        got = out[:, h * grp:(h + 1) * grp]
        rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
        assert float(rel.max()) <= 2e-3


def test_append_errors(ns):
    kf = torch.zeros((1, 256, 128), dtype=torch.float32, device="cuda")
    kv = ns.kv_nest_pack(kf, kf.clone())
    sh = ns.kv_shadow(kv)
    big = torch.zeros((1, 129, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ns.NestError, match="n <= block"):
        ns.kv_nest_append(kv, sh, big, big, 0)
    two = torch.zeros((1, 2, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ns.NestError, match="capacity"):
        ns.kv_nest_append(kv, sh, two, two, 255)


def test_append_near_ties_bit_exact(ns, oracle):
    # values on and around half-integer multiples of the block scale (and of
    # the refinement step), so that both codes are decided near a tie
    Hkv, d, block, cap = 2, 128, 128, 2 * 128
    kv, sh, okv, kf, vf = prefill(ns, oracle, Hkv, cap, d, block, 0, (529,))
    g = synth.rng(530)
    s0 = np.float32(0.37 / 7.0)
    def tie_values(n):
        q = g.integers(-7, 8, size=(Hkv, n, d)).astype(np.float32)
        half = g.choice(np.array([0.5, 0.03125, -0.5, -0.03125], np.float32), size=(Hkv, n, d))
        v = ((q + half) * s0).astype(np.float32)
        for _ in range(2):
            v = np.where(g.random(v.shape) < 0.3, np.nextafter(v, np.float32(np.inf)), v)
            v = np.where(g.random(v.shape) < 0.3, np.nextafter(v, np.float32(-np.inf)), v)
        v = np.clip(v, -7 * s0, 7 * s0).astype(np.float32)
        v[:, 0, 0] = 7 * s0
        return v
    pos = 0
    for n in (9, 5, 100, 17):
        nk, nv = tie_values(n), tie_values(n)
        ns.kv_nest_append(kv, sh, dev(nk), dev(nv), pos)
        oracle.kv_append(okv, kf, vf, nk, nv, pos)
        same(kv, okv)
        pos += n
