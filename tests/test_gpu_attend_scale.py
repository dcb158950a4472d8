"""kv_nest_attend against the oracle at magnitudes far from 1 (GPU).

The nested cache stores exact integer codes with fp32 block scales (BitNest,
Figure 4), so the attention output is defined for K, V and q of any
magnitude within fp32's range. The kernels pass only exact integers and
values in [0, 1] through f16: the query row is scaled by a power of two,
and the V block scale is applied in fp32. These cases cover tiny V (whose
products with softmax weights would be f16 subnormals), large K and V
(peaked softmax), queries beyond f16's largest finite value and far below
its normal range, and a transitional regime where many tokens share the
weight. Both views, both kernels (the wave kernel for up to 16 query rows
per kv head, the LDS-table kernel for more) and one 32K shape; each is held
to the normwise 2e-3 bound against the oracle's fp64 attention.
"""
from __future__ import annotations

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


def rel_err(o, ref):
    return float(np.max(np.linalg.norm(o - ref, axis=-1) / np.linalg.norm(ref, axis=-1)))


def queries(nq, Hq, d, key, std, positive=False):
    x = synth.normal((nq, Hq, d), key, std)
    return synth.to_bf16_bits(np.abs(x) if positive else x)


# (q std, K std, V std, all-positive queries)
SCALES = {
    "v1e-3": (1.0, 1.0, 1e-3, False),
    "v1e-4": (1.0, 1.0, 1e-4, False),
    "v1e-6": (1.0, 1.0, 1e-6, False),
    "kv30": (1.0, 30.0, 30.0, False),
    "q100": (100.0, 1.0, 1.0, False),
    "q1e5": (1e5, 1.0, 1.0, False),
    "q1e-3": (1e-3, 1.0, 1.0, False),
    "q1e-6_k1e-6": (1e-6, 1e-6, 1.0, False),
    "qk3": (3.0, 3.0, 1.0, False),
    "q_positive": (1.0, 1.0, 1.0, True),
    "q_positive3": (3.0, 1.0, 1.0, True),
}


@pytest.mark.parametrize("view", [0, 1])
@pytest.mark.parametrize("nq", [1, 9])  # 4 query rows per kv head (wave kernel), 36 (LDS tables)
@pytest.mark.parametrize("case", list(SCALES))
def test_kv_attend_at_scale(ns, oracle, case, nq, view):
    qs, ks, vs, pos = SCALES[case]
    Hq, Hkv, d, cap, ctx = 8, 2, 128, 2048, 1900
    ci = list(SCALES).index(case)
    kf, vf = synth.kv(Hkv, cap, d, (240, ci), ks, vs)
    q = queries(nq, Hq, d, (241, ci, nq), qs, pos)
    okv = oracle.kv_nest_pack(kf, vf)
    ref = oracle.kv_attend(q, okv, ctx, view)
    kv = ns.kv_nest_pack(dev(kf), dev(vf))
    out = host(ns.kv_nest_attend(dev(q.view(np.int16)), kv, ctx, view))
    assert np.all(np.isfinite(out))
    err = rel_err(out, ref)
    print(f"{case} nq={nq} view={view}: normwise {err:.3g}")
    assert err <= 2e-3, err


@pytest.mark.parametrize("view,nq,case", [(0, 1, "v1e-4"), (1, 9, "v1e-4"), (0, 1, "q100"),
                                          (1, 9, "q1e-3")])
def test_kv_attend_32k_at_scale(ns, oracle, view, nq, case):
    qs, ks, vs, pos = SCALES[case]
    Hq, Hkv, d, ctx = 32, 8, 128, 32768
    cap = ctx + 128
    grp = Hq // Hkv
    kf, vf = synth.kv(Hkv, cap, d, (242, view), ks, vs)
    q = queries(nq, Hq, d, (243, nq), qs, pos)
    kv = ns.kv_nest_pack(dev(kf), dev(vf))
    out = host(ns.kv_nest_attend(dev(q.view(np.int16)), kv, ctx, view))
    for h in (0, 7):
        okv = oracle.kv_nest_pack(kf[h:h + 1], vf[h:h + 1])
        ref = oracle.kv_attend(np.ascontiguousarray(q[:, h * grp:(h + 1) * grp]), okv, ctx, view)
        err = rel_err(out[:, h * grp:(h + 1) * grp], ref)
        print(f"32K {case} nq={nq} view={view} head {h}: normwise {err:.3g}")
        assert err <= 2e-3, err
