"""GPU parity: the HIP path against the CPU oracle, element by element.

The bar:
  * packed planes, scales, int8 activations, int32 group sums, argmax
    indices, targets, accepted lengths and emitted tokens are bit-exact;
  * fp32 outputs on the exact-fold paths (argmax, verify_accept) are
    bit-identical to the oracle. Elsewhere they are within
    (G+2) * 2^-24 * sa * sum_g |s_g A_g| of the exact value. That is the
    rounding bound of any fold order and sits below 1e-5 relative for
    G <= 165;
  * attention outputs are within 2e-3 of the fp64 oracle, normwise per
    (query, head).
Shapes span several tiles plus a ragged tail. Every input comes from
nested_quantized_weights_amd.synth, and every expected value from oracle/.
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

    nestspec.lib()  # raises if the HIP library is missing
    return nestspec


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def tiled(ns, base, refine, scales):
    """The oracle's storage-format planes, moved to the GPU's tile layout by nest_tile."""
    return ns.nest_tile(dev(base), None if refine is None else dev(refine), dev(scales))


def bound_ok(y, sa, scales, acc, step):
    s = scales.astype(np.float64) * step
    terms = s[None] * acc.astype(np.float64)
    exact = sa.astype(np.float64)[:, None] * terms.sum(axis=2)
    A = sa.astype(np.float64)[:, None] * np.abs(terms).sum(axis=2)
    G = scales.shape[1]
    err = np.abs(y.astype(np.float64) - exact)
    return np.all(err <= (G + 2) * U32 * A + 1e-45), float(np.max(err / (A + 1e-300)))


# ---------------------------------------------------------------------------
# nest_pack / kv_nest_pack / act_quant: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,group", [(1, 128, 128), (37, 384, 128), (300, 3584, 128),
                                             (5, 64, 4), (3, 16384, 16384), (2, 8, 8)])
def test_nest_pack_bit_exact(ns, oracle, rows, cols, group):
    w = synth.weights(rows, cols, (200, rows, cols))
    if rows > 3:
        w[3, :group] = 0.0  # an all-zero group
    w[0, 1] = 3.0  # a group dominated by one large weight
    b, r, s = ns.nest_pack(dev(w), group=group)
    ob, orf, os_ = oracle.nest_pack(w, group=group)
    assert np.array_equal(host(b), ob)
    assert np.array_equal(host(r), orf)
    assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))


def test_nest_pack_hand_example(ns):
    import json, os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_hand_example.json")))
    b, r, s = ns.nest_pack(dev(np.array(ex["w"], np.float32)), group=ex["group"])
    assert host(b).tolist() == ex["base_bytes"]
    assert host(r).tolist() == ex["refine_bytes"]
    assert host(s).tolist() == ex["scales"]


@pytest.mark.parametrize("M,K", [(1, 128), (9, 3584), (144, 4096), (3, 1000)])
def test_act_quant_bit_exact(ns, oracle, M, K):
    x = synth.activations(M, K, (201, M, K))
    x[0, :7] = [127.0, -63.5, 0.5, -0.25, 2.5, -1.5, 0.0]  # ties
    if M > 1:
        x[1] = 0.0
    qa, sa = ns.nest_act_quant(dev(x))
    oq, osa = oracle.act_quant(x)
    assert np.array_equal(host(qa), oq)
    assert np.array_equal(host(sa).view(np.uint32), osa.view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(16, 128), (37, 384), (300, 3584), (5, 1280), (4097, 512)])
def test_nest_tile_bit_exact(ns, oracle, rows, cols):
    # nest_tile against the independent numpy permutation of the documented layout
    from formats import tile_plane, tile_scales

    w = synth.weights(rows, cols, (203, rows, cols))
    ob, orf, osc = oracle.nest_pack(w)
    t = tiled(ns, ob, orf, osc)
    assert np.array_equal(host(t.base), tile_plane(ob, rows, cols))
    assert np.array_equal(host(t.refine), tile_plane(orf, rows, cols))
    assert np.array_equal(host(t.scales).view(np.uint32), tile_scales(osc, rows, cols // 128).view(np.uint32))
    t1 = ns.nest_tile(dev(ob), None, dev(osc))  # base only
    assert t1.refine is None and np.array_equal(host(t1.base), host(t.base))


@pytest.mark.parametrize("Hkv,cap,d,block", [(1, 128, 128, 128), (8, 384, 128, 128), (2, 64, 16, 32)])
def test_kv_nest_pack_bit_exact(ns, oracle, Hkv, cap, d, block):
    kf, vf = synth.kv(Hkv, cap, d, (202, Hkv, cap))
    kv = ns.kv_nest_pack(dev(kf), dev(vf), block=block)
    o = oracle.kv_nest_pack(kf, vf, block=block)
    for name in ("k_base", "k_refine", "v_base", "v_refine"):
        assert np.array_equal(host(getattr(kv, name)), o[name]), name
    for name in ("k_scale", "v_scale"):
        assert np.array_equal(host(getattr(kv, name)).view(np.uint32), o[name].view(np.uint32))


# ---------------------------------------------------------------------------
# draft_gemv / verify_gemm
# ---------------------------------------------------------------------------

def _layer(oracle, N, K, M, key):
    w = synth.weights(N, K, (210,) + key)
    x = synth.activations(M, K, (211,) + key)
    base, refine, scales = oracle.nest_pack(w)
    qa, sa = oracle.act_quant(x)
    return base, refine, scales, qa, sa


GEMV_SHAPES = [(16, 128, 1), (33, 256, 5), (100, 384, 9), (4096, 4096, 1), (4097, 3584, 16),
               (3584, 18944, 1), (777, 1280, 5)]


@pytest.mark.parametrize("N,K,M", GEMV_SHAPES)
def test_draft_gemv(ns, oracle, N, K, M):
    base, _, scales, qa, sa = _layer(oracle, N, K, M, (N, K, M))
    oy, oacc = oracle.draft_gemv(qa, sa, base, scales, want_acc=True)
    W = tiled(ns, base, None, scales)
    y, acc = ns.draft_gemv(dev(qa), dev(sa), W, acc_dbg=True)
    assert np.array_equal(host(acc), oacc)
    ok, worst = bound_ok(host(y), sa, scales, oacc, 1.0)
    assert ok, worst
    # the argmax path folds exactly: y bit-identical, indices equal
    y2, am = ns.draft_gemv(dev(qa), dev(sa), W, argmax=True)
    assert np.array_equal(host(y2).view(np.uint32), oy.view(np.uint32))
    assert host(am).tolist() == [oracle.argmax(oy[m]) for m in range(M)]


@pytest.mark.parametrize("N,K,M", [(3000, 512, 20), (5000, 384, 144), (1500, 256, 150), (20000, 128, 33),
                                   (1499, 256, 40), (9001, 256, 40)])
def test_draft_gemv_over_16_rows(ns, oracle, N, K, M):
    # More than 16 rows (the drafts of more than 16 sequences): the batched
    # kernel over the base plane alone (its codes merge to 16 q_b, folded at
    # s/16), in launches of up to 144 rows, then the row argmaxes. The group
    # sums are exact, y within the fold's bound, each argmax the exact one
    # wherever the row's top two are apart by more than twice the bound, and
    # the fp32-input path gives the same products.
    base, _, scales, qa, sa = _layer(oracle, N, K, M, (N, K, M, 2))
    oy, oacc = oracle.draft_gemv(qa, sa, base, scales, want_acc=True)
    W = tiled(ns, base, None, scales)
    y, acc = ns.draft_gemv(dev(qa), dev(sa), W, acc_dbg=True)
    assert np.array_equal(host(acc), oacc)
    ok, worst = bound_ok(host(y), sa, scales, oacc, 1.0)
    assert ok, worst
    y2, am = ns.draft_gemv(dev(qa), dev(sa), W, argmax=True)
    y2 = host(y2)
    assert np.array_equal(y2.view(np.uint32), host(y).view(np.uint32))
    terms = scales.astype(np.float64)[None] * oacc.astype(np.float64)
    exact = sa.astype(np.float64)[:, None] * terms.sum(axis=2)
    tol = (scales.shape[1] + 2) * U32 * sa.astype(np.float64)[:, None] * np.abs(terms).sum(axis=2)
    am = host(am)
    for r in range(M):
        order = np.argsort(-exact[r], kind="stable")
        margin = 2 * tol[r].max()
        assert exact[r, am[r]] >= exact[r, order[0]] - margin, r
        if exact[r, order[0]] - exact[r, order[1]] > margin:
            assert am[r] == order[0], r
        assert am[r] == int(np.argmax(y2[r]))  # the argmax of the kernel's own logits, lowest index first
    x = synth.activations(M, K, (211, N, K, M, 2))  # the activations _layer quantized
    yx = ns.draft_gemv_x(dev(x), W)
    assert np.array_equal(host(yx).view(np.uint32), host(y).view(np.uint32))
    # the row argmax reads 16 bytes at a time only where the rows allow it:
    # N = 1499 or 9001 and a caller's y 4 bytes off a 16-byte boundary take
    # the scalar loads, with the same results; rows are split into chunks
    # where there are few rows of many logits (20000 x 33 rows: 9 chunks,
    # 9001 x 40: 4, 5000 x 144: 2)
    yo = torch.empty(M * N + 1, dtype=torch.float32, device="cuda")[1:].view(M, N)
    assert yo.data_ptr() % 16 != 0
    y3, am3 = ns.draft_gemv(dev(qa), dev(sa), W, y=yo, argmax=True)
    assert np.array_equal(host(y3).view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(host(am3), am)


# M > 16 runs the batched kernel: (200, 2048, 144) and (1000, 1024, 144)
# split each row block's activation rows over 9 blocks (one column tile
# each); K = 128 leaves one part of a block's groups empty; (130, 384, 100)
# has an odd group count and ragged row and activation tiles; (5511, 256,
# 144) has more row blocks than three parts of them fit in one round, so it
# takes two-tile blocks (345 tiles, the last one partial). Few row blocks
# over 64 groups or more split the groups over four blocks per row block
# (the workspace path): (640, 8192, 144) with whole tiles; (300, 9216, 37)
# with a ragged last tile and three-part blocks; (200, 8320, 100) with 65
# groups (slices of 16, 16, 16 and 17); (130, 16384, 150) in two launches
# (144 + 6 rows) that share the workspace. More tiles than four per CU take
# five- to seven-tile blocks in one round: (17000, 256, 64) five (ragged
# last tile), (24000, 128, 50) six, (28672, 128, 144) seven. (4400, 8192,
# 20) splits the groups over three blocks for each of 69 row blocks (more
# counters than a 256-byte area holds; ragged last tile). A single weight
# row: (1, 256, 20) in one block, (1, 8192, 144) split over four slices.
# (30000, 256, 144): more tiles than seven rounds' worth of CUs, seven-tile
# blocks in two rounds; (28705, 128, 70) the same with a one-row last tile
# and ragged rows.
BATCHED_SHAPES = [(50, 512, 17), (200, 256, 144), (64, 384, 150), (200, 2048, 144), (1000, 1024, 144),
                  (64, 128, 33), (130, 384, 100), (5511, 256, 144),
                  (640, 8192, 144), (300, 9216, 37), (200, 8320, 100), (130, 16384, 150),
                  (17000, 256, 64), (24000, 128, 50), (28672, 128, 144), (4400, 8192, 20), (1, 256, 20),
                  (1, 8192, 144), (30000, 256, 144), (28705, 128, 70)]


@pytest.mark.parametrize("N,K,M", GEMV_SHAPES + BATCHED_SHAPES)
def test_verify_gemm(ns, oracle, N, K, M):
    base, refine, scales, qa, sa = _layer(oracle, N, K, M, (N, K, M, 1))
    oy, oacc = oracle.verify_gemm(qa, sa, base, refine, scales, want_acc=True)
    W = tiled(ns, base, refine, scales)
    y, acc = ns.verify_gemm(dev(qa), dev(sa), W, acc_dbg=True)
    assert np.array_equal(host(acc), oacc)
    ok, worst = bound_ok(host(y), sa, scales, oacc, 1.0 / 16)
    assert ok, worst
    y_nodbg = ns.verify_gemm(dev(qa), dev(sa), W)
    assert np.array_equal(host(y_nodbg).view(np.uint32), host(y).view(np.uint32))


@pytest.mark.parametrize("N,K", [(300, 4096), (300, 9216)])
def test_batched_verify_repeats(ns, oracle, N, K):
    # the batched kernel keeps no state between calls (the group split's
    # counters return to zero): calls in a row agree bit for bit, also after
    # calls with other shapes on the same stream and workspace
    base, refine, scales, qa, sa = _layer(oracle, N, K, 144, (11,))
    W = tiled(ns, base, refine, scales)
    y1 = host(ns.verify_gemm(dev(qa), dev(sa), W))
    b2, r2, s2, qa2, sa2 = _layer(oracle, 70, 1024, 40, (12,))
    b3, r3, s3, qa3, sa3 = _layer(oracle, 900, 8192, 20, (13,))
    ns.verify_gemm(dev(qa2), dev(sa2), tiled(ns, b2, r2, s2))
    for _ in range(3):
        ns.verify_gemm(dev(qa3), dev(sa3), tiled(ns, b3, r3, s3))
        y2 = host(ns.verify_gemm(dev(qa), dev(sa), W))
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    oy, oacc = oracle.verify_gemm(qa, sa, base, refine, scales, want_acc=True)
    ok, worst = bound_ok(y1, sa, scales, oacc, 1.0 / 16)
    assert ok, worst


def test_shapes_and_entry_points_share_one_workspace(ns, oracle):
    # The workspace starts with a counter zone that holds only block
    # counters, at the same offsets for every entry point and shape. A group
    # split over 69 row blocks (4400 x 8192, three slices), one over 10 row
    # blocks and four slices (640 x 8192), the fp32-input path of the first
    # shape, an argmax GEMV and the argmaxes of a 144-row draft (two chunks
    # per row, meeting through the zone's row counters) take turns on one
    # workspace, and each gives
    # bit for bit what it gives on a fresh one; the zone is zero afterwards.
    # (With the counters placed before the partial sums at a shape-dependent
    # offset, the 4-slice call's sums landed on the 69-row-block call's
    # counters.)
    la = _layer(oracle, 4400, 8192, 144, (14,))
    lb = _layer(oracle, 640, 8192, 144, (15,))
    Wa, Wb = tiled(ns, *la[:3]), tiled(ns, *lb[:3])
    x = dev(synth.activations(144, 8192, (16,)))
    L = ns.lib()
    zone = 4352
    assert L.verify_gemm_workspace_size(144, 8192, 4400) > zone
    assert L.verify_gemm_workspace_size(144, 8192, 640) > zone
    n = max(L.verify_gemm_workspace_size(144, 8192, 4400), L.verify_gemm_workspace_size(144, 8192, 640),
            L.nest_gemv_x_workspace_size(144, 8192, 4400), L.nest_gemv_x_workspace_size(1, 8192, 4400),
            L.draft_gemv_workspace_size(144, 4400))

    def fresh():
        return torch.zeros(n, dtype=torch.uint8, device="cuda")

    calls = {
        "split3": lambda ws: ns.verify_gemm(dev(la[3]), dev(la[4]), Wa, ws=ws),
        "split4": lambda ws: ns.verify_gemm(dev(lb[3]), dev(lb[4]), Wb, ws=ws),
        "x": lambda ws: ns.verify_gemm_x(x, Wa, ws=ws),
        "argmax": lambda ws: ns.draft_gemv_x(x[:1], Wa, argmax=True, want_y=False, ws=ws),
        "rows": lambda ws: ns.draft_gemv(dev(la[3]), dev(la[4]), Wa, argmax=True, want_y=False, ws=ws)[1],
    }
    ref = {k: host(f(fresh())) for k, f in calls.items()}
    ws = fresh()
    for k in ["split4", "split3", "rows", "split4", "x", "split3", "argmax", "rows", "split4", "x", "split3",
              "rows"]:
        got = host(calls[k](ws))
        assert np.array_equal(got.view(np.uint32), ref[k].view(np.uint32)), k
    assert not host(ws[:zone]).any()


def test_gemv_deterministic(ns, oracle):
    base, refine, scales, qa, sa = _layer(oracle, 3584, 18944, 5, (9,))
    args = [dev(qa), dev(sa), tiled(ns, base, refine, scales)]
    y1 = host(ns.verify_gemm(*args))
    y2 = host(ns.verify_gemm(*args))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_draft_reads_only_base_plane(ns, oracle):
    # BitNest Fig. 3: the draft never touches the refinement plane, and with
    # the refinement zeroed verify equals draft bit for bit (exact paths).
    base, refine, scales, qa, sa = _layer(oracle, 300, 512, 1, (10,))
    yd, _ = ns.draft_gemv(dev(qa), dev(sa), tiled(ns, base, None, scales), argmax=True)
    out = ns.verify_accept(dev(qa), dev(sa), 1, 0, tiled(ns, base, np.zeros_like(refine), scales),
                           dev(np.zeros(0, np.int32)), want_y=True)
    assert np.array_equal(host(yd).view(np.uint32), host(out["y"]).view(np.uint32))


# ---------------------------------------------------------------------------
# verify_accept: LM head + argmax + greedy accept
# ---------------------------------------------------------------------------

def test_table1_worked_round_on_gpu(ns, oracle):
    import json, os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "table1_round.json")))
    vocab = ex["vocab"]
    ids = {t: i for i, t in enumerate(vocab)}
    k, V, K = ex["k"], len(vocab), 128
    w = np.zeros((V, K), np.float32)
    w[np.arange(V), np.arange(V)] = 1.0
    x = np.zeros((k + 1, K), np.float32)
    for i, t in enumerate(ex["target_choices"]):
        x[i, ids[t]] = 1.0
    W = ns.nest_pack_tiled(dev(w))
    qa, sa = ns.nest_act_quant(dev(x))
    draft = dev(np.array([ids[t] for t in ex["draft"]], np.int32))
    out = ns.verify_accept(qa, sa, 1, k, W, draft)
    n = int(host(out["n_emitted"])[0])
    assert n == ex["expected_n_emitted"]
    assert [vocab[t] for t in host(out["emitted"])[0][:n]] == ex["expected_emitted"]


@pytest.mark.parametrize("V,K,B,k,alpha", [(1000, 256, 1, 8, 0.66), (4099, 512, 1, 4, 0.95),
                                           (2500, 384, 2, 3, 0.58), (640, 128, 1, 0, 0.5),
                                           (20000, 3584, 1, 15, 0.9)])
def test_verify_accept(ns, oracle, V, K, B, k, alpha):
    w = synth.weights(V, K, (220, V, K))
    x = synth.activations(B * (k + 1), K, (221, V, K))
    base, refine, scales = oracle.nest_pack(w)
    qa, sa = oracle.act_quant(x)
    t_ref = oracle.verify_gemm(qa, sa, base, refine, scales).argmax(axis=1).reshape(B, k + 1)
    draft = synth.plant_drafts(t_ref, alpha, V, (222, V))
    o = oracle.verify_accept(qa, sa, B, k, base, refine, scales, draft, want_y=True)
    W = tiled(ns, base, refine, scales)
    for rep in range(3):  # also checks the workspace is left ready for the next call
        g = ns.verify_accept(dev(qa), dev(sa), B, k, W,
                             dev(draft.reshape(-1) if k else np.zeros(0, np.int32)), want_y=True)
        assert np.array_equal(host(g["target"]), o["target"])
        assert np.array_equal(host(g["n_emitted"]), o["n_emitted"])
        assert np.array_equal(host(g["emitted"]), o["emitted"])
        assert np.array_equal(host(g["y"]).view(np.uint32), o["y"].view(np.uint32))


@pytest.mark.parametrize("V,K,B,k", [(5000, 512, 2, 8), (3000, 384, 1, 16), (20000, 1024, 16, 8),
                                     (1200, 256, 1, 150), (3001, 384, 3, 8),
                                     (20001, 384, 3, 8)])
def test_verify_accept_over_16_rows(ns, oracle, V, K, B, k):
    # More than 16 rows (several sequences, or k >= 16): the batched kernel
    # writes y (int32 group sums exact, the fp32 fold within its rounding
    # bound, in the batched kernel's order), then a per-row argmax and the
    # accept rule. A row's target is the exact argmax wherever the exact
    # logits' two largest are further apart than twice the bound, and
    # within that of the largest elsewhere; the rule's outputs follow
    # exactly from the targets, and the lengths advance by the emitted
    # counts. 151 rows take two batched launches (144 + 7). The row argmax
    # splits a row into chunks where there are few rows of many logits
    # (5000 x 18 rows: 2, 20000 x 144 rows: 8, 20001 x 27 rows: 9 chunks,
    # whose keys meet through a row counter); rows of 3001 and 20001
    # logits take its scalar loads.
    M = B * (k + 1)
    w = synth.weights(V, K, (224, V, K))
    x = synth.activations(M, K, (225, V, K))
    base, refine, scales = oracle.nest_pack(w)
    qa, sa = oracle.act_quant(x)
    oy, oacc = oracle.verify_gemm(qa, sa, base, refine, scales, want_acc=True)
    draft = synth.plant_drafts(oy.argmax(axis=1).reshape(B, k + 1), 0.8, V, (226, V))
    W = tiled(ns, base, refine, scales)
    length = torch.full((B,), 100, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    g = ns.verify_accept(dev(qa), dev(sa), B, k, W, dev(draft.reshape(-1)), length=length, next_token=nxt)
    y = host(g["y"])
    ok, worst = bound_ok(y, sa, scales, oacc, 1.0 / 16)
    assert ok, worst
    terms = (scales.astype(np.float64) / 16)[None] * oacc.astype(np.float64)
    exact = sa.astype(np.float64)[:, None] * terms.sum(axis=2)
    tol = (scales.shape[1] + 2) * U32 * sa.astype(np.float64)[:, None] * np.abs(terms).sum(axis=2)
    tg = host(g["target"]).reshape(-1)
    unique = 0
    for r in range(M):
        order = np.argsort(-exact[r], kind="stable")
        top, second = order[0], order[1]
        margin = 2 * tol[r].max()
        assert exact[r, tg[r]] >= exact[r, top] - margin, r
        if exact[r, top] - exact[r, second] > margin:
            assert tg[r] == top, r
            unique += 1
    assert unique >= M - 2
    n_got, em_got = host(g["n_emitted"]), host(g["emitted"])
    t2 = tg.reshape(B, k + 1)
    for b in range(B):
        a = 0
        while a < k and draft[b, a] == t2[b, a]:
            a += 1
        assert n_got[b] == a + 1
        assert list(em_got[b]) == list(t2[b, :a + 1]) + [-1] * (k - a)
        assert host(nxt)[b] == t2[b, a]  # the next round's input: the last emitted token
    assert np.array_equal(host(length), 100 + n_got)
    if M <= 18:  # the fp32-input path quantizes first: the same codes, the same logits
        gx = ns.verify_accept_x(dev(x), B, k, W, dev(draft.reshape(-1)))
        assert np.array_equal(host(gx["y"]).view(np.uint32), y.view(np.uint32))
        assert np.array_equal(host(gx["target"]).reshape(-1), tg)


def test_argmax_ties_take_lowest_index(ns, oracle):
    # Two identical LM-head rows tie on every logit: the lower index wins.
    V, K = 500, 256
    w = synth.weights(V, K, (223,))
    w[300] = w[77]
    w[77] *= 10.0
    w[300] = w[77]
    base, refine, scales = oracle.nest_pack(w)
    x = w[77:78].copy()
    qa, sa = oracle.act_quant(x)
    _, am = ns.draft_gemv(dev(qa), dev(sa), tiled(ns, base, None, scales), argmax=True)
    oy = oracle.draft_gemv(qa, sa, base, scales)
    assert int(host(am)[0]) == oracle.argmax(oy[0]) == 77


# ---------------------------------------------------------------------------
# kv_nest_attend
# ---------------------------------------------------------------------------

def _rel_err(o, ref):
    num = np.linalg.norm(o - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / den))


# Up to 16 query rows per kv head run the wave kernel: one 128-token block
# per wave up to 2048 blocks in all (32/8 heads at ctx 20000: 1256), several
# past that (8/8 heads at ctx 40000: 2504 blocks, two per wave).
@pytest.mark.parametrize("view", [0, 1])
@pytest.mark.parametrize("Hq,Hkv,cap,ctx,nq", [(32, 8, 256, 256, 1), (32, 8, 384, 300, 9),
                                               (28, 4, 512, 389, 5), (4, 1, 128, 1, 1),
                                               (8, 8, 1024, 1000, 8), (16, 2, 2048, 2048, 8),
                                               (32, 8, 20096, 20000, 1), (8, 8, 40960, 40000, 1),
                                               (28, 4, 512, 389, 12), (32, 8, 384, 300, 20)])
def test_kv_attend(ns, oracle, view, Hq, Hkv, cap, ctx, nq):
    # the last two have more than 64 query rows per kv head (84, 80): they
    # run in chunks of 9 and 16 queries
    d = 128
    kf, vf = synth.kv(Hkv, cap, d, (230, Hq, cap))
    q = synth.queries_bf16(nq, Hq, d, (231, Hq, nq))
    okv = oracle.kv_nest_pack(kf, vf)
    ref = oracle.kv_attend(q, okv, ctx, view)
    kv = ns.kv_nest_pack(dev(kf), dev(vf))
    out = host(ns.kv_nest_attend(dev(q.view(np.int16)), kv, ctx, view))
    assert _rel_err(out, ref) <= 2e-3
    if nq * (Hq // Hkv) > 64:  # the chunks with the length on the device (offset 5 on the host)
        length = torch.tensor([ctx - 5], dtype=torch.int32, device="cuda")
        out_d = host(ns.kv_nest_attend(dev(q.view(np.int16)), kv, 5, view, ctx_dev=length))
        assert _rel_err(out_d, ref) <= 2e-3


@pytest.mark.parametrize("view", [0, 1])
@pytest.mark.parametrize("nq", [5, 1])  # 20 query rows per kv head (LDS tables) and 4 (wave kernel)
def test_kv_attend_ignores_entries_past_ctx(ns, oracle, view, nq):
    Hkv, Hq, cap, d, ctx = 2, 8, 512, 128, 300
    kf, vf = synth.kv(Hkv, cap, d, (232,))
    q = dev(synth.queries_bf16(nq, Hq, d, (233,)).view(np.int16))
    kv = ns.kv_nest_pack(dev(kf), dev(vf))
    ref = host(ns.kv_nest_attend(q, kv, ctx, view))
    # poison every plane byte past ctx (K token-major, V dim-major per block)
    g = synth.rng(234)
    kb = kv.k_base.view(Hkv, cap, d // 2)
    kr = kv.k_refine.view(Hkv, cap, d // 2)
    kb[:, ctx:] = dev(g.integers(0, 256, size=(Hkv, cap - ctx, d // 2), dtype=np.uint8))
    kr[:, ctx:] = dev(g.integers(0, 256, size=(Hkv, cap - ctx, d // 2), dtype=np.uint8))
    for t in (kv.v_base, kv.v_refine):
        v = t.view(Hkv, cap // 128, d, 64)
        b0, t0 = divmod(ctx, 128)
        v[:, b0, :, t0 // 2:] = dev(g.integers(0, 256, size=(Hkv, d, 64 - t0 // 2), dtype=np.uint8))
        v[:, b0 + 1:] = dev(g.integers(0, 256, size=(Hkv, cap // 128 - b0 - 1, d, 64), dtype=np.uint8))
    kv.k_scale[:, (ctx + 127) // 128:] = 1e30
    kv.v_scale[:, (ctx + 127) // 128:] = 1e30
    out = host(ns.kv_nest_attend(q, kv, ctx, view))
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_kv_attend_deterministic(ns):
    kf, vf = synth.kv(8, 4096, 128, (235,))
    q = dev(synth.queries_bf16(9, 32, 128, (236,)).view(np.int16))
    kv = ns.kv_nest_pack(dev(kf), dev(vf))
    a = host(ns.kv_nest_attend(q, kv, 4000, 1))
    b = host(ns.kv_nest_attend(q, kv, 4000, 1))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------------------
# error paths through the C ABI (host-side validation)
# ---------------------------------------------------------------------------

def test_errors_are_reported(ns):
    qa = torch.zeros((1, 200), dtype=torch.int8, device="cuda")
    sa = torch.zeros(1, dtype=torch.float32, device="cuda")
    W = ns.Tiled(torch.zeros(1600, dtype=torch.uint8, device="cuda"), None,
                 torch.zeros(64, dtype=torch.float32, device="cuda"), 16, 200)
    with pytest.raises(ns.NestError, match="multiple of 128"):
        ns.draft_gemv(qa, sa, W)
    qa = torch.zeros((17, 128), dtype=torch.int8, device="cuda")
    W = ns.nest_tile(torch.zeros((16, 64), dtype=torch.uint8, device="cuda"), None,
                     torch.zeros((16, 1), dtype=torch.float32, device="cuda"))
    # more than 16 rows go through the batched kernel, which writes y: a
    # call that gives only the argmax output is refused on the host
    L = ns.lib()
    am = torch.zeros(17, dtype=torch.int32, device="cuda")
    ws = torch.zeros(L.draft_gemv_workspace_size(17, 16), dtype=torch.uint8, device="cuda")
    rc = L.draft_gemv(qa.data_ptr(), torch.zeros(17, dtype=torch.float32, device="cuda").data_ptr(), 17, 128,
                      W.base.data_ptr(), W.scales.data_ptr(), 16, 128, None, am.data_ptr(), None,
                      ws.data_ptr(), ws.numel(), None)
    assert rc == 1 and b"need y" in L.nest_last_error()
    with pytest.raises(ns.NestError, match="Tiled"):
        ns.draft_gemv(qa[:1], sa, torch.zeros((16, 64), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ns.NestError, match="multiple of 128"):
        ns.nest_tile(torch.zeros((16, 100), dtype=torch.uint8, device="cuda"), None,
                     torch.zeros((16, 1), dtype=torch.float32, device="cuda"))
