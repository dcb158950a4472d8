"""verify_accept_x_static: the verify pass with the accept step on the
library's own per-device scratch, for callers that cannot allocate (GPU).

It must give exactly what verify_accept_x gives with a caller workspace
(targets, accepted count, emitted tokens, logits, the advanced length and
the next input), on calls in a row that share the scratch: a large call,
then a smaller one, then one whose activations are quantized first into the
scratch. A call that needs more scratch than the array holds is refused on
the host.
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


def run_both(ns, V, K, B, k, key):
    W = ns.nest_pack_tiled(dev(synth.weights(V, K, (key, 0))))
    x = dev(synth.activations(B * (k + 1), K, (key, 1)))
    t = ns.verify_accept_x(x, B, k, W, torch.zeros(max(B * k, 1), dtype=torch.int32, device="cuda"))
    target = host(t["target"])
    draft = dev(synth.plant_drafts(target, 0.7, V, (key, 2)).ravel().astype(np.int32))
    outs = []
    for fn in (ns.verify_accept_x, ns.verify_accept_x_static):
        length = torch.full((B,), 1000, dtype=torch.int32, device="cuda")
        nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        o = fn(x, B, k, W, draft, want_y=True, length=length, next_token=nxt)
        outs.append({**{n: host(v) for n, v in o.items()}, "length": host(length), "next": host(nxt)})
    return outs


@pytest.mark.parametrize("first,second", [((152064, 3584, 1, 8), (4096, 512, 2, 3))])
def test_static_scratch_matches_the_workspace_call(ns, first, second):
    # a large call, a smaller one (the shared scratch keeps the first call's
    # keys past the second's), then quantize-first (16 rows of 16384 exceed
    # the in-kernel limit, so the codes go through the scratch too)
    for i, (V, K, B, k) in enumerate((first, second, (3000, 16384, 4, 3))):
        a, b = run_both(ns, V, K, B, k, 700 + i)
        for name in ("target", "n_emitted", "emitted", "length", "next"):
            assert np.array_equal(a[name], b[name]), (i, name)
        assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32)), i
        assert np.array_equal(b["length"], 1000 + b["n_emitted"])
        n = b["n_emitted"]
        assert np.all((n >= 1) & (n <= k + 1))
        assert np.array_equal(b["next"], b["emitted"][np.arange(B), n - 1])


def test_static_scratch_refuses_what_does_not_fit(ns):
    W = ns.Tiled(torch.zeros(16, dtype=torch.uint8, device="cuda"), torch.zeros(16, dtype=torch.uint8,
                 device="cuda"), torch.zeros(64, dtype=torch.float32, device="cuda"), 1 << 24, 65536)
    x = torch.zeros((16, 65536), dtype=torch.float32, device="cuda")
    with pytest.raises(ns.NestError, match="scratch"):
        ns.verify_accept_x_static(x, 2, 7, W, torch.zeros(14, dtype=torch.int32, device="cuda"))
