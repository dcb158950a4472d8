"""GPU parity at the configured full sizes, in the launch configuration bench.py times.

Every expected value comes from the oracle, which packs its own planes from
the same seeded fp32 weights. Nothing the GPU produced is fed to the oracle.
Where the oracle cannot cover a whole tensor in seconds, it runs on sampled
output rows, or on sampled kv heads (heads are independent). The bar is the
same as in test_gpu_parity.py.
  * linear_4096: 4096x4096, draft 1 row, verify 5 rows, checked in full.
  * qwen2.5-7b_layer: every linear of the layer on 512 sampled rows.
  * qwen2.5-7b_lm_head: the full 152064-row head with k = 8. verify_accept
    is checked in full on a pool of activation sets. Then 10k rounds with
    drafts planted at 0.58 / 0.66 / 0.95: every round's accepted length
    matches the accept rule on the same drafts, and the mean matches Eq. (1).
  * llama3-8b_batched_verify: the five distinct linears of one layer at
    144 rows, on 256 sampled rows each.
  * kv_32k: 32 q / 8 kv heads, 32768 context; draft (1 query, base view) and
    verify (9 queries, full view), on 2 sampled kv heads and their 8 q heads.
"""
import numpy as np
import pytest
import torch

from nested_quantized_weights_amd import synth

pytestmark = pytest.mark.gpu
U32 = 2.0 ** -24


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


def bound_ok(y, sa, scales, acc, step):
    s = scales.astype(np.float64) * step
    terms = s[None] * acc.astype(np.float64)
    exact = sa.astype(np.float64)[:, None] * terms.sum(axis=2)
    A = sa.astype(np.float64)[:, None] * np.abs(terms).sum(axis=2)
    err = np.abs(y.astype(np.float64) - exact)
    return bool(np.all(err <= (scales.shape[1] + 2) * U32 * A + 1e-45))


def check_linear(ns, oracle, w, x_draft, x_verify, rows):
    """GPU path on the full matrix; oracle on the sampled rows (its own packing)."""
    N, K = w.shape
    wd = dev(w)
    b, r, s = ns.nest_pack(wd)
    del wd
    ob, orf, osc = oracle.nest_pack(w[rows])
    assert np.array_equal(host(b[dev(rows)]), ob)
    assert np.array_equal(host(r[dev(rows)]), orf)
    assert np.array_equal(host(s[dev(rows)]).view(np.uint32), osc.view(np.uint32))
    W = ns.nest_tile(b, r, s)
    del b, r, s
    for x, verify in ((x_draft, False), (x_verify, True)):
        qa, sa = ns.nest_act_quant(dev(x))
        oqa, osa = oracle.act_quant(x)
        assert np.array_equal(host(qa), oqa)
        if verify:
            y, acc = ns.verify_gemm(qa, sa, W, acc_dbg=True)
            oy, oacc = oracle.verify_gemm(oqa, osa, ob, orf, osc, want_acc=True)
            step = 1.0 / 16
        else:
            y, acc = ns.draft_gemv(qa, sa, W, acc_dbg=True)
            oy, oacc = oracle.draft_gemv(oqa, osa, ob, osc, want_acc=True)
            step = 1.0
        acc_h = host(acc)[:, rows]
        assert np.array_equal(acc_h, oacc)
        assert bound_ok(host(y)[:, rows], osa, osc, oacc, step)


def test_linear_4096_full(ns, oracle):
    wl = synth.WORKLOADS["linear_4096"]
    key = synth.WORKLOAD_KEY["linear_4096"]
    w = synth.weights(wl["N"], wl["K"], (key, 0))
    x = synth.activations(wl["verify_rows"], wl["K"], (key, 1))
    check_linear(ns, oracle, w, x[:1], x, np.arange(wl["N"]))


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_qwen_layer_linears(ns, oracle, name):
    wl = synth.WORKLOADS["qwen2.5-7b_layer"]
    key = synth.WORKLOAD_KEY["qwen2.5-7b_layer"]
    N, K = wl["linears"][name]
    li = list(wl["linears"]).index(name)
    w = synth.weights(N, K, (key, 0, li))
    xd = synth.activations(1, K, (key, 1, li))
    xv = synth.activations(wl["k"] + 1, K, (key, 2, li))
    rows = np.sort(synth.rng(key, 7, li).choice(N, size=512, replace=False))
    check_linear(ns, oracle, w, xd, xv, rows)


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down"])
def test_llama_batched_verify_144(ns, oracle, name):
    wl = synth.WORKLOADS["llama3-8b_batched_verify"]
    key = synth.WORKLOAD_KEY["llama3-8b_batched_verify"]
    N, K = wl["linears"][name]
    li = list(wl["linears"]).index(name)
    M = wl["sequences"] * wl["rows_per_seq"]
    w = synth.weights(N, K, (key, 0, 0, li))
    x = synth.activations(M, K, (key, 1, 0, li))
    rows = np.sort(synth.rng(key, 7, li).choice(N, size=256, replace=False))
    W = ns.nest_pack_tiled(dev(w))
    ob, orf, osc = oracle.nest_pack(w[rows])
    qa, sa = ns.nest_act_quant(dev(x))
    oqa, osa = oracle.act_quant(x)
    assert np.array_equal(host(qa), oqa)
    y, acc = ns.verify_gemm(qa, sa, W, acc_dbg=True)
    oy, oacc = oracle.verify_gemm(oqa, osa, ob, orf, osc, want_acc=True)
    assert np.array_equal(host(acc)[:, rows], oacc)
    assert bound_ok(host(y)[:, rows], osa, osc, oacc, 1.0 / 16)
    y2 = ns.verify_gemm(qa, sa, W)  # the bench's launch (no debug output)
    assert np.array_equal(host(y2).view(np.uint32), host(y).view(np.uint32))


@pytest.fixture(scope="module")
def lm_head(ns, oracle):
    wl = synth.WORKLOADS["qwen2.5-7b_lm_head"]
    key = synth.WORKLOAD_KEY["qwen2.5-7b_lm_head"]
    V, K, k = wl["V"], wl["K"], wl["k"]
    w = synth.weights(V, K, (key, 0))
    ob, orf, osc = oracle.nest_pack(w)
    wd = dev(w)
    b, r, s = ns.nest_pack(wd)
    del wd, w
    assert np.array_equal(host(b), ob) and np.array_equal(host(r), orf)
    assert np.array_equal(host(s).view(np.uint32), osc.view(np.uint32))
    W = ns.nest_tile(b, r, s)
    del b, r, s
    pool, targets = [], []
    for p in range(4):  # activation sets whose full-vocabulary targets the oracle computes
        x = synth.activations(k + 1, K, (key, 1, p))
        oqa, osa = oracle.act_quant(x)
        pool.append((oqa, osa))
        targets.append(oracle.verify_gemm(oqa, osa, ob, orf, osc).argmax(axis=1))
    return {"o": (ob, orf, osc), "g": W, "pool": pool, "targets": np.stack(targets),
            "V": V, "k": k, "key": key}


def test_lm_head_verify_accept_full(ns, oracle, lm_head):
    ob, orf, osc = lm_head["o"]
    W = lm_head["g"]
    k, V = lm_head["k"], lm_head["V"]
    for p, (oqa, osa) in enumerate(lm_head["pool"][:2]):
        t = lm_head["targets"][p].reshape(1, k + 1)
        draft = synth.plant_drafts(t, 0.95, V, (lm_head["key"], 2, p))
        o = oracle.verify_accept(oqa, osa, 1, k, ob, orf, osc, draft, want_y=True)
        g = ns.verify_accept(dev(oqa), dev(osa), 1, k, W, dev(draft.ravel()), want_y=True)
        assert np.array_equal(host(g["target"]), o["target"])
        assert np.array_equal(host(g["n_emitted"]), o["n_emitted"])
        assert np.array_equal(host(g["emitted"]), o["emitted"])
        assert np.array_equal(host(g["y"]).view(np.uint32), o["y"].view(np.uint32))
        # the draft's own choice: base plane only, exact fold, same tie rule
        yd, am = ns.draft_gemv(dev(oqa[:1]), dev(osa[:1]), W, argmax=True)
        oyd = oracle.draft_gemv(oqa[:1], osa[:1], ob, osc)
        assert np.array_equal(host(yd).view(np.uint32), oyd.view(np.uint32))
        assert int(host(am)[0]) == oracle.argmax(oyd[0])


@pytest.mark.parametrize("alpha", [0.58, 0.66, 0.95])
def test_lm_head_planted_rounds_eq1(ns, oracle, lm_head, alpha):
    ob, orf, osc = lm_head["o"]
    W = lm_head["g"]
    k, V, key = lm_head["k"], lm_head["V"], lm_head["key"]
    R = synth.WORKLOADS["qwen2.5-7b_lm_head"]["rounds"]
    pool, targets = lm_head["pool"], lm_head["targets"]
    which = np.arange(R) % len(pool)
    drafts = synth.plant_drafts(targets[which], alpha, V, (key, 3, int(alpha * 100)))
    expect = np.array([oracle.accept(drafts[i], targets[which[i]])[0] for i in range(R)])
    qa_d = [dev(qa) for qa, _ in pool]
    sa_d = [dev(sa) for _, sa in pool]
    d_d = dev(drafts)
    n_d = torch.empty(R, dtype=torch.int32, device="cuda")
    out = {"target": torch.empty((1, k + 1), dtype=torch.int32, device="cuda"),
           "emitted": torch.empty((1, k + 1), dtype=torch.int32, device="cuda")}
    for i in range(R):
        out["n_emitted"] = n_d[i:i + 1]
        ns.verify_accept(qa_d[which[i]], sa_d[which[i]], 1, k, W, d_d[i], out=out)
    got = host(n_d)
    assert np.array_equal(got, expect)
    assert got.min() >= 1 and got.max() <= k + 1
    E = (1 - alpha ** (k + 1)) / (1 - alpha)
    p = np.array([alpha ** j * (1 - alpha) for j in range(k)] + [alpha ** k])
    sd = float(np.sqrt((np.arange(1, k + 2) ** 2) @ p - E ** 2))
    assert abs(got.mean() - E) < 4 * sd / np.sqrt(R)


@pytest.mark.parametrize("view,nq", [(0, 1), (1, 9)])
def test_kv_32k_sampled_heads(ns, oracle, view, nq):
    wl = synth.WORKLOADS["kv_32k"]
    key = synth.WORKLOAD_KEY["kv_32k"]
    Hq, Hkv, d, ctx = wl["q_heads"], wl["kv_heads"], wl["head_dim"], wl["context"]
    cap = ctx + 128
    grp = Hq // Hkv
    kf, vf = synth.kv(Hkv, cap, d, (key, 0))
    q = synth.queries_bf16(nq, Hq, d, (key, 1, nq))
    kv = ns.kv_nest_pack(dev(kf), dev(vf))
    out = host(ns.kv_nest_attend(dev(q.view(np.int16)), kv, ctx, view))
    for h in (0, 5):
        okv = oracle.kv_nest_pack(kf[h:h + 1], vf[h:h + 1])
        for name in ("k_base", "k_refine", "v_base", "v_refine"):
            n = okv[name].size
            assert np.array_equal(host(getattr(kv, name))[h * n:(h + 1) * n], okv[name])
        ref = oracle.kv_attend(np.ascontiguousarray(q[:, h * grp:(h + 1) * grp]), okv, ctx, view)
        got = out[:, h * grp:(h + 1) * grp]
        rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
        assert float(rel.max()) <= 2e-3, float(rel.max())
