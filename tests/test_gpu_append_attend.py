"""kv_nest_append_attend_exact: a verify pass's append and exact attention in
one call (the append folded into the open-block kernel) must leave the
output, the planes, the scales and the shadows bit-identical to
kv_nest_append followed by kv_nest_attend_exact ("How Speculative Decoding
Speeds Up Inference", section "Drafting and checking tokens", step 2).

Cases: a pass inside one block, one that crosses a block boundary, one that
starts at a block boundary (no old tokens in the block), one that ends at a
block's last token, one at an empty cache, one query (the append alone,
then the one-query launch), GQA widths 7, 4 and 1, both views, host and
device positions, and a device position whose append would not fit (nothing
appended, as kv_nest_append).
"""
import numpy as np
import pytest
import torch

from nested_quantized_weights_amd import synth

pytestmark = pytest.mark.gpu


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


def prefilled(ns, kf, vf, ctx0):
    kd, vd = dev(kf), dev(vf)
    kv = ns.kv_nest_pack(kd, vd)
    sh = ns.kv_shadow(kv)
    ns.kv_nest_shadow_fill(kv, kd, vd, ctx0, sh)
    return kv, sh


def state(kv, sh):
    """Every byte the append may write: planes, scales (bits) and shadows (bits)."""
    out = [host(t).view(np.uint8).ravel() for t in (kv.k_base, kv.k_refine, kv.v_base, kv.v_refine)]
    out += [host(t).view(np.uint32).ravel() for t in (kv.k_scale, kv.v_scale, sh[0], sh[1])]
    return out


# (Hq, Hkv, capacity, ctx0, n)
CASES = [(28, 4, 1024, 300, 5), (28, 4, 1024, 126, 5), (28, 4, 1024, 128, 5), (28, 4, 1024, 379, 5),
         (16, 4, 512, 0, 9), (28, 4, 512, 200, 1), (28, 4, 512, 255, 2), (16, 16, 640, 250, 9),
         (8, 2, 384, 120, 17)]


@pytest.mark.parametrize("view", [0, 1])
@pytest.mark.parametrize("on_device", [False, True])
@pytest.mark.parametrize("Hq,Hkv,cap,ctx0,n", CASES)
def test_fused_equals_append_then_attend(ns, Hq, Hkv, cap, ctx0, n, on_device, view):
    key = 900 + ctx0 + n
    kf, vf = synth.kv(Hkv, cap, 128, (key, 0))
    kf[:, ctx0:] = 0.0
    vf[:, ctx0:] = 0.0
    kn, vn = synth.kv(Hkv, n, 128, (key, 1))
    q = dev(synth.queries_bf16(n, Hq, 128, (key, 2)).view(np.int16))
    length = torch.full((1,), ctx0, dtype=torch.int32, device="cuda") if on_device else None
    base = 0 if on_device else ctx0
    kv, sh = prefilled(ns, kf, vf, ctx0)
    ns.kv_nest_append(kv, sh, dev(kn), dev(vn), base, pos_dev=length)
    ref = host(ns.kv_nest_attend_exact(q, kv, sh, base + n, view, ctx_dev=length))
    kv2, sh2 = prefilled(ns, kf, vf, ctx0)
    got = host(ns.kv_nest_append_attend_exact(q, kv2, sh2, dev(kn), dev(vn), base, view, pos_dev=length))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    for a, b in zip(state(kv2, sh2), state(kv, sh)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("view", [0, 1])
def test_fused_append_that_does_not_fit(ns, view):
    # a device position with the pass reaching past the capacity: neither
    # path appends, and both attend over the (clamped) visible length
    Hq, Hkv, cap, n = 28, 4, 512, 5
    ctx0 = cap - 2
    kf, vf = synth.kv(Hkv, cap, 128, (931, 0))
    kn, vn = synth.kv(Hkv, n, 128, (931, 1))
    q = dev(synth.queries_bf16(n, Hq, 128, (931, 2)).view(np.int16))
    length = torch.full((1,), ctx0, dtype=torch.int32, device="cuda")
    kv, sh = prefilled(ns, kf, vf, ctx0)
    before = state(kv, sh)
    ns.kv_nest_append(kv, sh, dev(kn), dev(vn), 0, pos_dev=length)
    ref = host(ns.kv_nest_attend_exact(q, kv, sh, n, view, ctx_dev=length))
    kv2, sh2 = prefilled(ns, kf, vf, ctx0)
    got = host(ns.kv_nest_append_attend_exact(q, kv2, sh2, dev(kn), dev(vn), 0, view, pos_dev=length))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    for a, b, c in zip(state(kv2, sh2), state(kv, sh), before):
        assert np.array_equal(a, b) and np.array_equal(a, c)


def test_fused_rounds_in_a_row(ns):
    # verify passes back to back on one cache, the length advancing on the
    # device by a different count each time, against the two-call sequence
    Hq, Hkv, cap = 28, 4, 1024
    kf, vf = synth.kv(Hkv, cap, 128, (941, 0))
    kf[:, 100:] = 0.0
    vf[:, 100:] = 0.0
    kv, sh = prefilled(ns, kf, vf, 100)
    kv2, sh2 = prefilled(ns, kf, vf, 100)
    L = torch.full((1,), 100, dtype=torch.int32, device="cuda")
    L2 = L.clone()
    for r, adv in enumerate([5, 1, 3, 5, 2, 5, 4]):
        kn, vn = synth.kv(Hkv, 5, 128, (942, r))
        q = dev(synth.queries_bf16(5, Hq, 128, (943, r)).view(np.int16))
        ns.kv_nest_append(kv, sh, dev(kn), dev(vn), 0, pos_dev=L)
        ref = host(ns.kv_nest_attend_exact(q, kv, sh, 5, 1, ctx_dev=L))
        got = host(ns.kv_nest_append_attend_exact(q, kv2, sh2, dev(kn), dev(vn), 0, 1, pos_dev=L2))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), r
        L += adv
        L2 += adv
    for a, b in zip(state(kv2, sh2), state(kv, sh)):
        assert np.array_equal(a, b)
