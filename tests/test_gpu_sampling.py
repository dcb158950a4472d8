"""GPU parity of speculative sampling (nest_sample, verify_sample) against
the oracle ("How Speculative Decoding Speeds Up Inference", section "The
same output as the large model alone").

A draw is an integer decided by floating point: the kernels sum exponentials
in fp32 in their own order, the oracle in fp64 in id order. Where the
oracle's target lies more than DELTA (in probability) from the edges of the
id it draws, the kernel must draw the same id; closer to an edge, either id
whose interval lies within DELTA of the target is valid. Every draw is
checked that way (test_* asserts the interval condition for each), and each
test also counts exact agreement, which must hold for all but a few draws.

DELTA = 3e-5: exp2 of a rounded argument is within ~2e-6 relative of the
exact weight for |y - max| / T up to ~50 (larger gaps carry weights below
1e-21 of the total); the chunk sums, their prefix and the in-chunk prefix
add rounding of at most (11 + 75 + 11) * 2^-24 ~ 6e-6 of the running
weight; the residual max(0, p - q) subtracts two such values whose total is
at most 2. Accept tests compare u with p/q, each side within ~2e-5
relative, so a decision is checked exactly where |u - p/q| > RDELTA * p/q.
"""
import numpy as np
import pytest
import torch

from nested_quantized_weights_amd import synth

pytestmark = pytest.mark.gpu
DELTA = 3e-5
RDELTA = 1e-4


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


def within(lo, hi, tg):
    return lo - DELTA <= tg <= hi + DELTA


@pytest.mark.parametrize("M,V,T", [(1, 1000, 1.0), (5, 2049, 0.7), (16, 4096, 1.5), (3, 152064, 1.0),
                                   (2, 152064, 0.6), (4, 33, 1.0), (1, 1, 1.0), (2, 600000, 1.0)])
def test_sample_matches_oracle(ns, oracle, M, V, T):
    y = synth.logits(M, V, (730, M, V))
    yd = dev(y)
    exact = total = 0
    for rep in range(6):
        u = synth.uniforms(M, (731, M, V, rep))
        got = host(ns.sample(yd, T, dev(u)))
        for r in range(M):
            t = int(got[r])
            assert 0 <= t < V
            lo, hi, tg = oracle.sample_interval(y[r], T, u[r], t)
            assert within(lo, hi, tg), (r, t, lo, hi, tg)
            exact += t == oracle.sample(y[r], T, u[r])[0]
            total += 1
    assert exact >= total - max(1, total // 20)


def test_sample_masked_ids_and_extreme_uniforms(ns, oracle):
    V = 5000
    y = synth.logits(4, V, (732,))
    y[:, ::3] = -np.inf  # masked ids are never drawn
    y[3, :] = -np.inf
    y[3, 4321] = 0.5  # one live id
    for u0 in (0.0, 0.5, np.float32(0.99999994)):
        u = np.full(4, u0, np.float32)
        got = host(ns.sample(dev(y), 1.0, dev(u)))
        assert np.all(got % 3 != 0) and got[3] == 4321
        for r in range(3):
            lo, hi, tg = oracle.sample_interval(y[r], 1.0, u[r], int(got[r]))
            assert within(lo, hi, tg)


def test_sample_low_temperature_is_argmax(ns):
    y = synth.logits(8, 152064, (733,))
    got = host(ns.sample(dev(y), 1e-4, dev(synth.uniforms(8, (734,)))))
    assert np.array_equal(got, y.argmax(axis=1))


def round_inputs(oracle, B, k, V, T, key, noise=0.3):
    yt = synth.logits(B * (k + 1), V, key).reshape(B, k + 1, V)
    yd = synth.logits_near(yt[:, :k], key + (1,), noise=noise)
    ud = synth.uniforms((B, max(k, 1)), key + (2,))
    draft = np.array([[oracle.sample(yd[b, i], T, ud[b, i])[0] for i in range(k)] for b in range(B)],
                     np.int32).reshape(B, k)
    u_acc = synth.uniforms((B, k), key + (3,))
    u_fin = synth.uniforms(B, key + (4,))
    return yt, yd, draft, u_acc, u_fin


def check_round(oracle, yt, yd, draft, T, u_acc, u_fin, n_got, em_got):
    """Every decision valid within the rounding bands; returns whether the
    round equals the oracle's exactly."""
    k = yt.shape[0] - 1
    n_o, em_o, ratio, _ = oracle.verify_sample(yt, yd, draft, T, u_acc, u_fin)
    a = int(n_got) - 1
    assert 0 <= a <= k
    assert list(em_got[:a]) == list(draft[:a])
    assert list(em_got[a + 1:]) == [-1] * (k - a)
    for i in range(a):  # kept: u < p/q, up to rounding
        assert u_acc[i] < ratio[i] * (1 + RDELTA), (i, u_acc[i], ratio[i])
    if a < k:  # rejected: u >= p/q, up to rounding
        assert u_acc[a] >= ratio[a] * (1 - RDELTA), (a, u_acc[a], ratio[a])
    t = int(em_got[a])
    assert 0 <= t < yt.shape[1]
    lo, hi, tg = oracle.final_interval(yt, yd, T, a, u_fin, t)
    assert within(lo, hi, tg), (a, t, lo, hi, tg)
    return int(n_got) == n_o and np.array_equal(em_got, em_o)


@pytest.mark.parametrize("B,k,V,T,noise", [(1, 4, 1000, 1.0, 0.3), (3, 1, 2049, 0.8, 1.0), (2, 8, 4096, 1.0, 0.3),
                                           (1, 8, 152064, 1.0, 0.3), (2, 4, 152064, 0.7, 0.1),
                                           (4, 0, 5000, 1.0, 0.3), (1, 32, 700, 1.2, 0.5),
                                           (1, 2, 600000, 1.0, 0.3), (2, 9, 3000, 1.0, 0.3)])
def test_verify_sample_matches_oracle(ns, oracle, B, k, V, T, noise):
    exact = total = 0
    for rep in range(3):
        yt, yd, draft, u_acc, u_fin = round_inputs(oracle, B, k, V, T, (740, B, k, V, rep), noise)
        out = ns.verify_sample(dev(yt), dev(yd) if k else None, dev(draft), T, dev(u_acc), dev(u_fin))
        n, em = host(out["n_emitted"]), host(out["emitted"])
        for b in range(B):
            exact += check_round(oracle, yt[b], yd[b], draft[b], T, u_acc[b], u_fin[b], n[b], em[b])
            total += 1
    assert exact >= total - max(1, total // 10)


def test_verify_sample_planted_outcomes(ns, oracle):
    # u_acc = 0 keeps every draft with p(d) > 0; identical models keep all;
    # a draft id outside the vocabulary is rejected; identical models with
    # u_acc = 1 reject with no residual mass and draw from p
    B, k, V = 4, 5, 3000
    yt, yd, draft, u_acc, u_fin = round_inputs(oracle, B, k, V, 1.0, (745,))
    u_acc[0] = 0.0
    yd[1] = yt[1, :k]
    draft[2, 2] = V + 7
    yd[3] = yt[3, :k]
    u_acc[3, 0] = 1.0
    out = ns.verify_sample(dev(yt), dev(yd), dev(draft), 1.0, dev(u_acc), dev(u_fin))
    n, em = host(out["n_emitted"]), host(out["emitted"])
    assert n[0] == k + 1 and n[1] == k + 1 and n[2] <= 3 and n[3] == 1
    for b in range(B):
        check_round(oracle, yt[b], yd[b], draft[b], 1.0, u_acc[b], u_fin[b], n[b], em[b])


def test_verify_sample_errors(ns):
    V = 100
    yt = torch.zeros((1, 34, V), dtype=torch.float32, device="cuda")
    yd = torch.zeros((1, 33, V), dtype=torch.float32, device="cuda")
    dr = torch.zeros((1, 33), dtype=torch.int32, device="cuda")
    ua = torch.zeros((1, 33), dtype=torch.float32, device="cuda")
    uf = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ns.NestError, match="k=33"):
        ns.verify_sample(yt, yd, dr, 1.0, ua, uf)
    with pytest.raises(ns.NestError, match="temperature"):
        ns.verify_sample(yt[:, :2], yd[:, :1], dr[:, :1], 0.0, ua[:, :1], uf)
    with pytest.raises(ns.NestError, match="workspace"):
        ns.verify_sample(yt[:, :2], yd[:, :1], dr[:, :1], 1.0, ua[:, :1], uf,
                         ws=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ns.NestError, match="temperature"):
        ns.sample(yt[0], float("nan"), torch.zeros(34, dtype=torch.float32, device="cuda"))


def tiled(ns, base, refine, scales):
    return ns.nest_tile(dev(base), dev(refine), dev(scales))


@pytest.mark.parametrize("V,K,k,T", [(20000, 1024, 4, 0.1), (5003, 512, 8, 0.05)])
def test_sampled_round_from_the_nested_head(ns, oracle, V, K, k, T):
    # The draft's logits come from the base plane (draft_gemv_x), the
    # target's from both planes (verify_accept_x); both on their exact-fold
    # paths, so the logits equal the oracle's bit for bit. Draft i and
    # target row i see the same hidden state x_i (a synthetic stand-in).
    w = synth.weights(V, K, (750, V, K))
    x = synth.activations(k + 1, K, (751, V, K))
    base, refine, scales = oracle.nest_pack(w)
    W = tiled(ns, base, refine, scales)
    u_d = synth.uniforms(k, (752, V))
    u_acc = synth.uniforms((1, k), (753, V))
    u_fin = synth.uniforms(1, (754, V))
    yd_rows, drafts = [], []
    for i in range(k):
        qa, sa = oracle.act_quant(x[i:i + 1])
        oy = oracle.draft_gemv(qa, sa, base, scales)
        gy, _ = ns.draft_gemv_x(dev(x[i:i + 1]), W, argmax=True)
        assert np.array_equal(host(gy).view(np.uint32), oy.view(np.uint32))
        t = int(host(ns.sample(gy, T, dev(u_d[i:i + 1])))[0])
        lo, hi, tg = oracle.sample_interval(oy[0], T, u_d[i], t)
        assert within(lo, hi, tg)
        yd_rows.append(oy[0])
        drafts.append(oracle.sample(oy[0], T, u_d[i])[0])
    yd = np.stack(yd_rows)[None]
    draft = np.array([drafts], np.int32)
    qa, sa = oracle.act_quant(x)
    oy_t = oracle.verify_accept(qa, sa, 1, k, base, refine, scales, draft, want_y=True)["y"]
    out = ns.verify_accept_x(dev(x), 1, k, W, dev(draft), want_y=True)
    gy_t = out["y"]
    assert np.array_equal(host(gy_t).view(np.uint32), oy_t.view(np.uint32))
    res = ns.verify_sample(gy_t.view(1, k + 1, V), dev(yd), dev(draft), T, dev(u_acc), dev(u_fin))
    n, em = host(res["n_emitted"]), host(res["emitted"])
    check_round(oracle, oy_t, yd[0], draft[0], T, u_acc[0], u_fin[0], n[0], em[0])
