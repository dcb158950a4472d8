"""kv_nest_attend_exact: the k+1 queries of a verify pass in one launch, each
seeing the cache as a one-token pass at its own position would (GPU).

After one kv_nest_append of the nq new tokens, query i's output must be
bit-identical to the one-query kv_nest_attend a position-by-position pass
makes (append token i, attend with query i), and within the 2e-3 normwise
tolerance of the oracle's position-by-position attention ("How Speculative
Decoding Speeds Up Inference", section "Drafting and checking tokens",
step 2; BitNest, Figure 4). Cases cross a block boundary inside the pass,
start at an empty cache, use every GQA width the configurations have, both
views, and device-held lengths; one runs at the 32K context.
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


def inputs(Hq, Hkv, cap, ctx0, nq, key, k_std=1.0, v_std=1.0, q_std=1.0):
    kf, vf = synth.kv(Hkv, cap, 128, (key, 0), k_std, v_std)
    kf[:, ctx0:] = 0.0
    vf[:, ctx0:] = 0.0
    kn, vn = synth.kv(Hkv, nq, 128, (key, 1), k_std, v_std)
    q = synth.queries_bf16(nq, Hq, 128, (key, 2), q_std)
    return kf, vf, kn, vn, q


# (Hq, Hkv, capacity, ctx0, nq). A workgroup packs floor(16 / (Hq/Hkv))
# queries (2 for GQA 7 or 8, 4 for GQA 4, 16 for GQA 1). The last three: one
# query (the entry point's one-query path), 9 queries of a GQA group of 8
# (72 rows, more than kv_nest_attend's 64), and 17 queries of GQA 1 (a full
# group of 16 and one more) crossing a block boundary
CASES = [(28, 4, 1024, 300, 5), (8, 2, 512, 126, 5), (32, 8, 384, 250, 9), (4, 1, 256, 0, 3),
         (16, 16, 640, 511, 2), (28, 4, 512, 123, 9), (28, 4, 512, 200, 1), (64, 8, 512, 380, 9),
         (16, 16, 640, 370, 17)]


@pytest.mark.parametrize("view", [0, 1])
@pytest.mark.parametrize("on_device", [False, True])
@pytest.mark.parametrize("Hq,Hkv,cap,ctx0,nq", CASES)
def test_exact_equals_position_by_position(ns, oracle, Hq, Hkv, cap, ctx0, nq, on_device, view):
    kf, vf, kn, vn, q = inputs(Hq, Hkv, cap, ctx0, nq, 250 + ctx0)
    qd = dev(q.view(np.int16))
    length = torch.full((1,), ctx0, dtype=torch.int32, device="cuda") if on_device else None
    base = 0 if on_device else ctx0
    # one append of all nq tokens, then one exact launch
    kv, sh = prefilled(ns, kf, vf, ctx0)
    ns.kv_nest_append(kv, sh, dev(kn), dev(vn), base, pos_dev=length)
    got = host(ns.kv_nest_attend_exact(qd, kv, sh, base + nq, view, ctx_dev=length))
    # position by position: append token i, attend with query i
    kv2, sh2 = prefilled(ns, kf, vf, ctx0)
    ref = np.empty_like(got)
    for i in range(nq):
        ns.kv_nest_append(kv2, sh2, dev(kn[:, i:i + 1]), dev(vn[:, i:i + 1]), base + i, pos_dev=length)
        ref[i] = host(ns.kv_nest_attend(qd[i:i + 1], kv2, base + i + 1, view, ctx_dev=length))[0]
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the oracle, position by position
    okv = oracle.kv_nest_pack(kf, vf)
    ok, ov = kf.copy(), vf.copy()
    for i in range(nq):
        oracle.kv_append(okv, ok, ov, kn[:, i:i + 1], vn[:, i:i + 1], ctx0 + i)
        o = oracle.kv_attend(np.ascontiguousarray(q[i:i + 1]), okv, ctx0 + i + 1, view)[0]
        rel = np.linalg.norm(got[i] - o, axis=-1) / np.linalg.norm(o, axis=-1)
        assert float(rel.max()) <= 2e-3, (i, float(rel.max()))


def test_exact_at_32k_crossing_a_block(ns):
    Hq, Hkv, nq = 28, 4, 5
    ctx0 = 32768 - 2
    cap = 32768 + 256
    kf, vf, kn, vn, q = inputs(Hq, Hkv, cap, ctx0, nq, 260)
    qd = dev(q.view(np.int16))
    kv, sh = prefilled(ns, kf, vf, ctx0)
    ns.kv_nest_append(kv, sh, dev(kn), dev(vn), ctx0)
    got = host(ns.kv_nest_attend_exact(qd, kv, sh, ctx0 + nq, 1))
    kv2, sh2 = prefilled(ns, kf, vf, ctx0)
    for i in range(nq):
        ns.kv_nest_append(kv2, sh2, dev(kn[:, i:i + 1]), dev(vn[:, i:i + 1]), ctx0 + i)
        ref = host(ns.kv_nest_attend(qd[i:i + 1], kv2, ctx0 + i + 1, 1))[0]
        assert np.array_equal(got[i].view(np.uint32), ref.view(np.uint32)), i


# (k_std, v_std, q_std): the magnitudes of the kv_nest_attend scale tests, here
# through the open-block rebuild of the exact pass
SCALES = [(1.0, 1e-4, 1.0), (1.0, 1e-3, 1.0), (30.0, 30.0, 1.0), (1.0, 1.0, 100.0), (1.0, 1.0, 1e-3),
          (1e-4, 1.0, 1.0)]


@pytest.mark.parametrize("view", [0, 1])
@pytest.mark.parametrize("k_std,v_std,q_std", SCALES)
def test_exact_at_extreme_scales(ns, oracle, k_std, v_std, q_std, view):
    Hq, Hkv, cap, ctx0, nq = 28, 4, 512, 250, 9
    kf, vf, kn, vn, q = inputs(Hq, Hkv, cap, ctx0, nq, 270, k_std, v_std, q_std)
    qd = dev(q.view(np.int16))
    kv, sh = prefilled(ns, kf, vf, ctx0)
    ns.kv_nest_append(kv, sh, dev(kn), dev(vn), ctx0)
    got = host(ns.kv_nest_attend_exact(qd, kv, sh, ctx0 + nq, view))
    okv = oracle.kv_nest_pack(kf, vf)
    ok, ov = kf.copy(), vf.copy()
    for i in range(nq):
        oracle.kv_append(okv, ok, ov, kn[:, i:i + 1], vn[:, i:i + 1], ctx0 + i)
        o = oracle.kv_attend(np.ascontiguousarray(q[i:i + 1]), okv, ctx0 + i + 1, view)[0]
        rel = np.linalg.norm(got[i] - o, axis=-1) / np.linalg.norm(o, axis=-1)
        assert float(rel.max()) <= 2e-3, (i, float(rel.max()))
