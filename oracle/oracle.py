"""Python access to the CPU oracle (oracle/nest_oracle.c).

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. It never imports the
HIP package, and the HIP package never imports it.

Each wrapper takes and returns numpy arrays and converts nothing but
dtypes and layout. All of the method's arithmetic is in the C file, which
cites the pages for each step.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnestoracle.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build  # noqa: WPS433 (local import on demand)

        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "oracle_set_threads": (None, [ctypes.c_int]),
        "oracle_get_threads": (ctypes.c_int, []),
        "oracle_quantize_group": (None, [_p, _i64, _p, _p, _p]),
        "oracle_pack_nibbles": (None, [_p, _i64, _p]),
        "oracle_unpack_nibbles": (None, [_p, _i64, _p]),
        "oracle_nest_pack": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _p]),
        "oracle_act_quant": (None, [_p, _i64, _i64, _p, _p]),
        "oracle_draft_gemv": (None, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _p, _p]),
        "oracle_verify_gemm": (None, [_p, _p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _p]),
        "oracle_argmax": (_i64, [_p, _i64]),
        "oracle_accept": (ctypes.c_int, [_p, _p, _i64, _p]),
        "oracle_verify_accept": (None, [_p, _p, _i64, _i64, _i64, _p, _p, _p, _i64, _i64,
                                        _p, _p, _p, _p, _p]),
        "oracle_kv_nest_pack": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _i64,
                                               _p, _p, _p, _p, _p, _p]),
        "oracle_expected_tokens": (ctypes.c_double, [ctypes.c_double, _i64]),
        "oracle_token_time": (ctypes.c_double, [ctypes.c_double, _i64, ctypes.c_double, ctypes.c_double]),
        "oracle_choose_k": (_i64, [ctypes.c_double, ctypes.c_double, _p, _i64]),
        "oracle_alpha_estimate": (ctypes.c_double, [_p, _p, _i64, ctypes.c_double, ctypes.c_double,
                                                    ctypes.c_double]),
        "oracle_sample": (_i64, [_p, _i64, ctypes.c_float, ctypes.c_float, _p]),
        "oracle_sample_interval": (None, [_p, _i64, ctypes.c_float, ctypes.c_float, _i64, _p, _p, _p]),
        "oracle_verify_sample": (_i64, [_p, _p, _i64, _i64, ctypes.c_float, _p, _p, ctypes.c_float,
                                        _p, _p, _p]),
        "oracle_final_interval": (None, [_p, _p, _i64, _i64, ctypes.c_float, _i64, ctypes.c_float, _i64,
                                         _p, _p, _p]),
        "oracle_kv_append": (ctypes.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                            _p, _p, _p, _p, _p, _p]),
        "oracle_kv_attend": (None, [_p, _i64, _i64, _i64, _i64, _i64, _i64,
                                    _p, _p, _p, _p, _p, _p, _i64, ctypes.c_int, _p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def quantize_group(w):
    w = _c(w, np.float32).ravel()
    qb = np.empty(w.size, np.int8)
    qr = np.empty(w.size, np.int8)
    s = np.zeros(1, np.float32)
    _load().oracle_quantize_group(_ptr(w), w.size, _ptr(qb), _ptr(qr), _ptr(s))
    return qb, qr, float(s[0])


def pack_nibbles(codes):
    codes = _c(codes, np.int8).ravel()
    plane = np.empty(codes.size // 2, np.uint8)
    _load().oracle_pack_nibbles(_ptr(codes), codes.size, _ptr(plane))
    return plane


def unpack_nibbles(plane, n=None):
    plane = _c(plane, np.uint8).ravel()
    n = plane.size * 2 if n is None else n
    codes = np.empty(n, np.int8)
    _load().oracle_unpack_nibbles(_ptr(plane), n, _ptr(codes))
    return codes


def nest_pack(w, group=128):
    w = _c(w, np.float32)
    rows, cols = w.shape
    base = np.empty((rows, cols // 2), np.uint8)
    refine = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // group), np.float32)
    rc = _load().oracle_nest_pack(_ptr(w), rows, cols, group, _ptr(base), _ptr(refine),
                                  _ptr(scales))
    if rc != 0:
        raise ValueError("oracle_nest_pack: bad sizes")
    return base, refine, scales


def act_quant(x):
    x = _c(x, np.float32)
    M, K = x.shape
    qa = np.empty((M, K), np.int8)
    sa = np.empty(M, np.float32)
    _load().oracle_act_quant(_ptr(x), M, K, _ptr(qa), _ptr(sa))
    return qa, sa


def draft_gemv(qa, sa, base, scales, group=128, want_acc=False):
    qa = _c(qa, np.int8)
    sa = _c(sa, np.float32)
    base = _c(base, np.uint8)
    scales = _c(scales, np.float32)
    M, K = qa.shape
    N = base.shape[0]
    y = np.empty((M, N), np.float32)
    acc = np.empty((M, N, K // group), np.int32) if want_acc else None
    _load().oracle_draft_gemv(_ptr(qa), _ptr(sa), M, K, _ptr(base), _ptr(scales), N, group,
                              _ptr(y), _ptr(acc))
    return (y, acc) if want_acc else y


def verify_gemm(qa, sa, base, refine, scales, group=128, want_acc=False):
    qa = _c(qa, np.int8)
    sa = _c(sa, np.float32)
    base = _c(base, np.uint8)
    refine = _c(refine, np.uint8)
    scales = _c(scales, np.float32)
    M, K = qa.shape
    N = base.shape[0]
    y = np.empty((M, N), np.float32)
    acc = np.empty((M, N, K // group), np.int32) if want_acc else None
    _load().oracle_verify_gemm(_ptr(qa), _ptr(sa), M, K, _ptr(base), _ptr(refine),
                               _ptr(scales), N, group, _ptr(y), _ptr(acc))
    return (y, acc) if want_acc else y


def argmax(y):
    y = _c(y, np.float32).ravel()
    return int(_load().oracle_argmax(_ptr(y), y.size))


def accept(draft, target):
    draft = _c(draft, np.int32).ravel()
    target = _c(target, np.int32).ravel()
    k = draft.size
    assert target.size == k + 1
    emitted = np.empty(k + 1, np.int32)
    n = _load().oracle_accept(_ptr(draft), _ptr(target), k, _ptr(emitted))
    return int(n), emitted


def verify_accept(qa, sa, B, k, base, refine, scales, draft, group=128, want_y=False):
    qa = _c(qa, np.int8)
    sa = _c(sa, np.float32)
    base = _c(base, np.uint8)
    refine = _c(refine, np.uint8)
    scales = _c(scales, np.float32)
    draft = _c(draft, np.int32).reshape(B, k)
    K = qa.shape[1]
    V = base.shape[0]
    assert qa.shape[0] == B * (k + 1)
    target = np.empty((B, k + 1), np.int32)
    n_emitted = np.empty(B, np.int32)
    emitted = np.empty((B, k + 1), np.int32)
    y = np.empty((B * (k + 1), V), np.float32) if want_y else None
    _load().oracle_verify_accept(_ptr(qa), _ptr(sa), B, k, K, _ptr(base), _ptr(refine),
                                 _ptr(scales), V, group, _ptr(draft), _ptr(target),
                                 _ptr(n_emitted), _ptr(emitted), _ptr(y))
    out = {"target": target, "n_emitted": n_emitted, "emitted": emitted}
    if want_y:
        out["y"] = y
    return out


def kv_nest_pack(kf, vf, block=128):
    kf = _c(kf, np.float32)
    vf = _c(vf, np.float32)
    Hkv, cap, d = kf.shape
    nb = cap // block
    kb = np.empty(Hkv * cap * d // 2, np.uint8)
    kr = np.empty_like(kb)
    vb = np.empty_like(kb)
    vr = np.empty_like(kb)
    ks = np.empty((Hkv, nb), np.float32)
    vs = np.empty((Hkv, nb), np.float32)
    rc = _load().oracle_kv_nest_pack(_ptr(kf), _ptr(vf), Hkv, cap, d, block, _ptr(kb),
                                     _ptr(kr), _ptr(ks), _ptr(vb), _ptr(vr), _ptr(vs))
    if rc != 0:
        raise ValueError("oracle_kv_nest_pack: bad sizes")
    return {"k_base": kb, "k_refine": kr, "k_scale": ks, "v_base": vb, "v_refine": vr,
            "v_scale": vs, "n_kv_heads": Hkv, "capacity": cap, "head_dim": d,
            "block": block}


def kv_append(kv, kf, vf, k_new, v_new, pos):
    """Append k_new / v_new [Hkv][n][d] at positions pos..pos+n-1 of the cache
    dict `kv` (planes and scales updated in place). kf / vf [Hkv][cap][d] are
    the oracle's fp32 values of every token and are updated too."""
    assert kf.dtype == np.float32 and kf.flags.c_contiguous and vf.dtype == np.float32
    kn = _c(k_new, np.float32)
    vn = _c(v_new, np.float32)
    Hkv, n, d = kn.shape
    rc = _load().oracle_kv_append(_ptr(kf), _ptr(vf), _ptr(kn), _ptr(vn), Hkv, kv["capacity"], d,
                                  kv["block"], int(pos), n, _ptr(kv["k_base"]), _ptr(kv["k_refine"]),
                                  _ptr(kv["k_scale"]), _ptr(kv["v_base"]), _ptr(kv["v_refine"]),
                                  _ptr(kv["v_scale"]))
    if rc != 0:
        raise ValueError("oracle_kv_append: bad sizes")
    return kv


def kv_attend(q_bf16, kv, ctx_len, view):
    q = _c(q_bf16, np.uint16)
    nq, Hq, d = q.shape
    assert d == kv["head_dim"]
    out = np.empty((nq, Hq, d), np.float64)
    _load().oracle_kv_attend(_ptr(q), nq, Hq, kv["n_kv_heads"], d, kv["capacity"],
                             kv["block"], _ptr(kv["k_base"]), _ptr(kv["k_refine"]),
                             _ptr(kv["k_scale"]), _ptr(kv["v_base"]), _ptr(kv["v_refine"]),
                             _ptr(kv["v_scale"]), int(ctx_len), int(view), _ptr(out))
    return out


def expected_tokens(alpha, k):
    """Eq. (1)."""
    return _load().oracle_expected_tokens(float(alpha), int(k))


def token_time(alpha, k, t_draft, t_pass):
    """Eq. (2)."""
    return _load().oracle_token_time(float(alpha), int(k), float(t_draft), float(t_pass))


def choose_k(alpha, t_draft, t_pass):
    """argmin_k Eq. (2) over k = 0 .. len(t_pass)-1 (t_pass[k]: pass time with k drafts)."""
    tp = _c(t_pass, np.float64)
    return int(_load().oracle_choose_k(float(alpha), float(t_draft), _ptr(tp), tp.size - 1))


def alpha_estimate(accepted, k, decay=1.0, prior_accepted=1.0, prior_rejected=1.0):
    a = _c(accepted, np.int64)
    kk = _c(np.broadcast_to(np.asarray(k, np.int64), a.shape), np.int64)
    return _load().oracle_alpha_estimate(_ptr(a), _ptr(kk), a.size, float(decay), float(prior_accepted),
                                         float(prior_rejected))


def sample(y, T, u):
    """One token from softmax(y / T) by inverse CDF with the uniform u:
    (token, margin of the decision from its interval's edges)."""
    yy = _c(y, np.float32).ravel()
    m = np.zeros(1, np.float64)
    t = _load().oracle_sample(_ptr(yy), yy.size, float(T), float(u), _ptr(m))
    return int(t), float(m[0])


def sample_interval(y, T, u, t):
    """Interval [lo, hi) of token t in the running sum of softmax(y / T), and the target u."""
    yy = _c(y, np.float32).ravel()
    out = np.zeros(3, np.float64)
    _load().oracle_sample_interval(_ptr(yy), yy.size, float(T), float(u), int(t), _ptr(out[0:]),
                                   _ptr(out[1:]), _ptr(out[2:]))
    return float(out[0]), float(out[1]), float(out[2])


def _spec_inputs(yt, yd, draft, u_acc):
    yt = _c(yt, np.float32)
    k1, V = yt.shape
    k = k1 - 1
    yd = _c(yd if k else np.zeros((1, V), np.float32), np.float32)
    dr = _c(np.asarray(draft, np.int32).reshape(-1) if k else np.zeros(1, np.int32), np.int32)
    ua = _c(np.asarray(u_acc, np.float32).reshape(-1) if k else np.zeros(1, np.float32), np.float32)
    return yt, yd, dr, ua, k, V


def verify_sample(yt, yd, draft, T, u_acc, u_fin):
    """Speculative-sampling round of one sequence: (n_emitted, emitted [k+1],
    ratio p/q of every slot [k], edge margin of the drawn token)."""
    yt, yd, dr, ua, k, V = _spec_inputs(yt, yd, draft, u_acc)
    em = np.empty(k + 1, np.int32)
    ratio = np.zeros(max(k, 1), np.float64)
    m = np.zeros(1, np.float64)
    n = _load().oracle_verify_sample(_ptr(yt), _ptr(yd), k, V, float(T), _ptr(dr), _ptr(ua), float(u_fin),
                                     _ptr(em), _ptr(ratio), _ptr(m))
    return int(n), em, ratio[:k], float(m[0])


def final_interval(yt, yd, T, a, u_fin, t):
    """Interval [lo, hi) of token t in the last token's distribution after a
    kept drafts (residual of slot a+1, or the bonus when a = k), and the target."""
    yt, yd, _, _, k, V = _spec_inputs(yt, yd, np.zeros(max(yt.shape[0] - 1, 1), np.int32),
                                      np.zeros(max(yt.shape[0] - 1, 1), np.float32))
    out = np.zeros(3, np.float64)
    _load().oracle_final_interval(_ptr(yt), _ptr(yd), k, V, float(T), int(a), float(u_fin), int(t),
                                  _ptr(out[0:]), _ptr(out[1:]), _ptr(out[2:]))
    return float(out[0]), float(out[1]), float(out[2])
