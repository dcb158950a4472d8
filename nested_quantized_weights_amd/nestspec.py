"""Python binding of libnestspec.so (include/nestspec.h).

Argument marshalling only. Tensors give device pointers, torch's current
stream gives the HIP stream, and every computation runs in the library's HIP
kernels. There is no CPU fallback. If the library is missing or a call
fails, NestError is raised.

torch is imported before the library is loaded, so the library binds to the
HIP runtime torch already loaded (same soname) and shares its device memory
and streams.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnestspec.so")


class NestError(RuntimeError):
    """A nestspec call returned an error status (or the library is missing)."""


def library_path() -> str:
    return _LIB_PATH


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_lib = None
_lock = threading.Lock()


class _KV(ctypes.Structure):
    _fields_ = [("k_base", _p), ("k_refine", _p), ("k_scale", _p), ("v_base", _p),
                ("v_refine", _p), ("v_scale", _p), ("n_kv_heads", _i64), ("head_dim", _i64),
                ("capacity", _i64), ("block", _i64)]


class _Alpha(ctypes.Structure):
    _fields_ = [("accepted", ctypes.c_double), ("rejected", ctypes.c_double), ("decay", ctypes.c_double)]


_d = ctypes.c_double

_SIGS = {
    "nest_last_error": (ctypes.c_char_p, []),
    "nest_pack": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "nest_act_quant": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p]),
    "draft_gemv": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _i64, _i64, _p, _p, _p, _p, _sz, _p]),
    "draft_gemv_workspace_size": (_sz, [_i64, _i64]),
    "verify_gemm": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _p, _p, _sz, _p]),
    "verify_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "verify_accept": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _p, _p,
                                     _p, _p, _p, _p, _p, _sz, _p]),
    "verify_accept_workspace_size": (_sz, [_i64, _i64, _i64]),
    "nest_tile": (ctypes.c_int, [_p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "nest_tile_plane_bytes": (_sz, [_i64, _i64]),
    "nest_tile_scale_count": (_sz, [_i64, _i64, _i64]),
    "draft_gemv_x": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _i64, _i64, _p, _p, _p, _sz, _p]),
    "verify_gemm_x": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _p, _sz, _p]),
    "verify_accept_x": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _p, _p,
                                       _p, _p, _p, _p, _p, _sz, _p]),
    "nest_gemv_x_workspace_size": (_sz, [_i64, _i64, _i64]),
    "verify_accept_x_static": (ctypes.c_int, [_p, _i64, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _p, _p,
                                              _p, _p, _p, _p, _p]),
    "kv_nest_pack": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p]),
    "nest_expected_tokens": (_d, [_d, _i64]),
    "nest_token_time": (_d, [_d, _i64, _d, _d]),
    "nest_choose_k": (_i64, [_d, _d, _p, _i64, ctypes.POINTER(_d)]),
    "nest_alpha_init": (None, [ctypes.POINTER(_Alpha), _d, _d, _d]),
    "nest_alpha_update": (None, [ctypes.POINTER(_Alpha), _i64, _i64]),
    "nest_alpha_value": (_d, [ctypes.POINTER(_Alpha)]),
    "kv_nest_append": (ctypes.c_int, [ctypes.POINTER(_KV), _p, _p, _p, _p, _p, _i64, _i64, _p]),
    "kv_nest_shadow_floats": (_sz, [_i64, _i64, _i64]),
    "kv_nest_shadow_fill": (ctypes.c_int, [ctypes.POINTER(_KV), _p, _p, _i64, _i64, _p, _p, _p]),
    "kv_nest_attend": (ctypes.c_int, [_p, _i64, _i64, ctypes.POINTER(_KV), _p, _i64, ctypes.c_int, _p,
                                      _p, _sz, _p]),
    "kv_nest_attend_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "kv_nest_attend_exact_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "kv_nest_attend_exact": (ctypes.c_int, [_p, _i64, _i64, ctypes.POINTER(_KV), _p, _p, _p, _i64, ctypes.c_int,
                                            _p, _p, _sz, _p]),
    "kv_nest_append_attend_exact": (ctypes.c_int, [_p, _i64, _i64, ctypes.POINTER(_KV), _p, _p, _p, _p, _p,
                                                   _i64, ctypes.c_int, _p, _p, _sz, _p]),
    "nest_sample": (ctypes.c_int, [_p, _i64, _i64, ctypes.c_float, _p, _p, _p, _sz, _p]),
    "nest_sample_workspace_size": (_sz, [_i64, _i64]),
    "verify_sample": (ctypes.c_int, [_p, _p, _i64, _i64, _i64, ctypes.c_float, _p, _p, _p, _p, _p, _p,
                                     _sz, _p]),
    "verify_sample_workspace_size": (_sz, [_i64, _i64, _i64]),
    "nest_embed": (ctypes.c_int, [_p, _i64, _i64, _p, _i64, _p, _p]),
    "nest_add_rmsnorm": (ctypes.c_int, [_p, _p, _p, _i64, _i64, ctypes.c_float, _p, _p]),
    "nest_rope_split": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _i64, _i64, ctypes.c_float, ctypes.c_int,
                                       _p, _p, _p, _p]),
    "nest_swiglu": (ctypes.c_int, [_p, _i64, _i64, _p, _p]),
    "nest_read_stream": (ctypes.c_int, [_p, _sz, _p, _p]),
}

SYMBOLS = tuple(_SIGS)


def lib():
    """Load libnestspec.so once (raises NestError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise NestError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                                "(hipcc for gfx950) first")
            handle = ctypes.CDLL(_LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib().nest_last_error().decode(errors="replace")
        raise NestError(f"{what} failed (status {rc}): {msg}")


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, what: str, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise NestError(f"{what}: {name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise NestError(f"{what}: {name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise NestError(f"{what}: {name} must be contiguous")
    return t


# Workspaces, cached per (device, stream, kind): calls on one stream run
# in order, so they can share one. They start all zero, as the GEMV
# workspaces must (each call leaves its block counter at zero again).
_ws_cache: dict = {}


def workspace(nbytes: int, device: torch.device, key: str) -> torch.Tensor:
    s = torch.cuda.current_stream(device).cuda_stream
    k = (device.index, s, key)
    t = _ws_cache.get(k)
    if t is None or t.numel() < nbytes:
        t = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[k] = t
    return t


def gemv_x_workspace(M: int, K: int, N: int, device: torch.device) -> torch.Tensor:
    """The zeroed workspace of the fp32-activation GEMV calls."""
    return workspace(lib().nest_gemv_x_workspace_size(M, K, N), device, "gemv")


def nest_pack(w: torch.Tensor, group: int = 128, out=None):
    """fp32 [rows][cols] -> (base uint8 [rows][cols/2], refine, scales fp32 [rows][cols/group])."""
    what = "nest_pack"
    _dev(w, torch.float32, what, "w")
    rows, cols = w.shape
    if out is None:
        out = (torch.empty((rows, cols // 2), dtype=torch.uint8, device=w.device),
               torch.empty((rows, cols // 2), dtype=torch.uint8, device=w.device),
               torch.empty((rows, cols // group), dtype=torch.float32, device=w.device))
    base, refine, scales = out
    _check(lib().nest_pack(_ptr(w), rows, cols, group, _ptr(base), _ptr(refine), _ptr(scales),
                           _stream(w.device)), what)
    return base, refine, scales


class Tiled:
    """A weight matrix in the tile layout (include/nestspec.h): what the
    draft / verify entry points read. rows and cols are the logical shape."""

    def __init__(self, base, refine, scales, rows, cols):
        self.base, self.refine, self.scales = base, refine, scales
        self.rows, self.cols = int(rows), int(cols)
        self.shape = (self.rows, self.cols)


def nest_tile(base, refine, scales, group: int = 128) -> Tiled:
    """Storage format (nest_pack's planes and scales) -> tile layout."""
    what = "nest_tile"
    _dev(base, torch.uint8, what, "base")
    if refine is not None:
        _dev(refine, torch.uint8, what, "refine")
    _dev(scales, torch.float32, what, "scales")
    rows, half = base.shape
    cols = 2 * half
    L = lib()
    nb = L.nest_tile_plane_bytes(rows, cols)
    ns = L.nest_tile_scale_count(rows, cols, group)
    if nb == 0 or ns == 0:
        raise NestError(f"{what}: unsupported shape rows={rows} cols={cols} group={group} "
                        "(the tile layout needs group 128 and cols a multiple of 128)")
    dev = base.device
    bt = torch.empty(nb, dtype=torch.uint8, device=dev)
    rt = torch.empty(nb, dtype=torch.uint8, device=dev) if refine is not None else None
    st = torch.empty(ns, dtype=torch.float32, device=dev)
    _check(L.nest_tile(_ptr(base), _ptr(refine), _ptr(scales), rows, cols, group, _ptr(bt), _ptr(rt),
                       _ptr(st), _stream(dev)), what)
    return Tiled(bt, rt, st, rows, cols)


def nest_pack_tiled(w: torch.Tensor, group: int = 128) -> Tiled:
    """nest_pack then nest_tile: a weight matrix ready for the draft / verify calls."""
    b, r, s = nest_pack(w, group)
    t = nest_tile(b, r, s, group)
    del b, r, s
    return t


def nest_act_quant(x: torch.Tensor, out=None):
    """fp32 [M][K] -> (qa int8 [M][K], sa fp32 [M])."""
    what = "nest_act_quant"
    _dev(x, torch.float32, what, "x")
    M, K = x.shape
    if out is None:
        out = (torch.empty((M, K), dtype=torch.int8, device=x.device),
               torch.empty(M, dtype=torch.float32, device=x.device))
    qa, sa = out
    _check(lib().nest_act_quant(_ptr(x), M, K, _ptr(qa), _ptr(sa), _stream(x.device)), what)
    return qa, sa


def _tiled(W, what, planes):
    if not isinstance(W, Tiled):
        raise NestError(f"{what}: weights must be a Tiled matrix (nest_tile / nest_pack_tiled)")
    if planes == 2 and W.refine is None:
        raise NestError(f"{what}: the refinement plane is missing")
    return W


def draft_gemv(qa, sa, W, group: int = 128, y=None, want_y: bool = True, argmax: bool = False,
               argmax_out=None, acc_dbg: bool = False, ws=None):
    """W4A8 over the base plane of W (Tiled). Returns y [M][N] (or None),
    plus argmax [M] when asked, plus the exact int32 group sums [M][N][G]
    when acc_dbg."""
    what = "draft_gemv"
    _dev(qa, torch.int8, what, "qa")
    _dev(sa, torch.float32, what, "sa")
    W = _tiled(W, what, 1)
    M, K = qa.shape
    N = W.rows
    dev = qa.device
    ret_y = y is not None or want_y or not argmax
    if y is None and (ret_y or M > 16):  # more than 16 rows: the library writes y on the way
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    am = None
    wsp, wsn = None, 0
    if argmax:
        am = argmax_out if argmax_out is not None else torch.empty(M, dtype=torch.int32, device=dev)
        if ws is None:
            ws = workspace(lib().draft_gemv_workspace_size(M, N), dev, "gemv")
        wsp, wsn = _ptr(ws), ws.numel()
    acc = torch.empty((M, N, K // group), dtype=torch.int32, device=dev) if acc_dbg else None
    _check(lib().draft_gemv(_ptr(qa), _ptr(sa), M, K, _ptr(W.base), _ptr(W.scales), N, group, _ptr(y),
                            _ptr(am), _ptr(acc), wsp, wsn, _stream(dev)), what)
    out = [y if ret_y else None]
    if argmax:
        out.append(am)
    if acc_dbg:
        out.append(acc)
    return out[0] if len(out) == 1 else tuple(out)


def verify_gemm(qa, sa, W, group: int = 128, y=None, acc_dbg: bool = False, ws=None):
    """W8A8 over both planes of W (Tiled). Returns y [M][N] (and the int32
    group sums when acc_dbg)."""
    what = "verify_gemm"
    _dev(qa, torch.int8, what, "qa")
    _dev(sa, torch.float32, what, "sa")
    W = _tiled(W, what, 2)
    M, K = qa.shape
    N = W.rows
    dev = qa.device
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N, K // group), dtype=torch.int32, device=dev) if acc_dbg else None
    wsn = lib().verify_gemm_workspace_size(M, K, N)
    if wsn and (ws is None or ws.numel() < wsn):
        ws = workspace(wsn, dev, "verify_gemm")
    _check(lib().verify_gemm(_ptr(qa), _ptr(sa), M, K, _ptr(W.base), _ptr(W.refine), _ptr(W.scales), N,
                             group, _ptr(y), _ptr(acc), _ptr(ws) if wsn else None, ws.numel() if wsn else 0,
                             _stream(dev)), what)
    return (y, acc) if acc_dbg else y


def _accept_out(B, k, V, dev, want_y):
    out = {"target": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
           "n_emitted": torch.empty(B, dtype=torch.int32, device=dev),
           "emitted": torch.empty((B, k + 1), dtype=torch.int32, device=dev)}
    if want_y:
        out["y"] = torch.empty((B * (k + 1), V), dtype=torch.float32, device=dev)
    return out


def verify_accept(qa, sa, B: int, k: int, W, draft, group: int = 128, want_y: bool = False, out=None,
                  ws=None, length=None, next_token=None):
    """Verify pass through the nested LM head W (Tiled) plus the greedy
    accept step. Returns a dict of device tensors: target [B][k+1],
    n_emitted [B], emitted [B][k+1] (and y when want_y). length (int32 [B],
    device) is advanced by n_emitted when given; next_token (int32 [B])
    receives the last emitted token."""
    what = "verify_accept"
    _dev(qa, torch.int8, what, "qa")
    _dev(sa, torch.float32, what, "sa")
    _dev(draft, torch.int32, what, "draft")
    W = _tiled(W, what, 2)
    K = qa.shape[1]
    V = W.rows
    dev = qa.device
    if out is None:
        out = _accept_out(B, k, V, dev, want_y or B * (k + 1) > 16)  # more rows: y holds the logits
    if ws is None:
        ws = workspace(lib().verify_accept_workspace_size(B, k, V), dev, "gemv")
    _check(lib().verify_accept(_ptr(qa), _ptr(sa), B, k, K, _ptr(W.base), _ptr(W.refine), _ptr(W.scales),
                               V, group, _ptr(draft), _ptr(out["target"]), _ptr(out["n_emitted"]),
                               _ptr(out["emitted"]), _ptr(out.get("y")), _ptr(length), _ptr(next_token),
                               _ptr(ws), ws.numel(), _stream(dev)), what)
    return out


def draft_gemv_x(x, W, group: int = 128, y=None, want_y: bool = True, argmax: bool = False,
                 argmax_out=None, ws=None):
    """draft_gemv on fp32 activations x [M][K], quantized inside the kernel.
    Returns y (or None), plus argmax [M] when asked."""
    what = "draft_gemv_x"
    _dev(x, torch.float32, what, "x")
    W = _tiled(W, what, 1)
    M, K = x.shape
    N = W.rows
    dev = x.device
    ret_y = y is not None or want_y or not argmax
    if y is None and (ret_y or M > 16):  # more than 16 rows: the library writes y on the way
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    am = None
    if argmax:
        am = argmax_out if argmax_out is not None else torch.empty(M, dtype=torch.int32, device=dev)
    if ws is None:
        ws = gemv_x_workspace(M, K, N, dev)
    _check(lib().draft_gemv_x(_ptr(x), M, K, _ptr(W.base), _ptr(W.scales), N, group, _ptr(y), _ptr(am),
                              _ptr(ws), ws.numel(), _stream(dev)), what)
    if argmax:
        return (y, am) if ret_y else am
    return y


def verify_gemm_x(x, W, group: int = 128, y=None, ws=None):
    """verify_gemm on fp32 activations x [M][K], quantized inside the kernel
    (or first into the workspace)."""
    what = "verify_gemm_x"
    _dev(x, torch.float32, what, "x")
    W = _tiled(W, what, 2)
    M, K = x.shape
    N = W.rows
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = gemv_x_workspace(M, K, N, x.device)
    _check(lib().verify_gemm_x(_ptr(x), M, K, _ptr(W.base), _ptr(W.refine), _ptr(W.scales), N, group,
                               _ptr(y), _ptr(ws), ws.numel(), _stream(x.device)), what)
    return y


def verify_accept_x(x, B: int, k: int, W, draft, group: int = 128, want_y: bool = False, out=None,
                    ws=None, length=None, next_token=None):
    """verify_accept on fp32 activations x [B*(k+1)][K], quantized inside the kernel."""
    what = "verify_accept_x"
    _dev(x, torch.float32, what, "x")
    _dev(draft, torch.int32, what, "draft")
    W = _tiled(W, what, 2)
    K = x.shape[1]
    V = W.rows
    dev = x.device
    if out is None:
        out = _accept_out(B, k, V, dev, want_y or B * (k + 1) > 16)  # more rows: y holds the logits
    if ws is None:
        ws = gemv_x_workspace(B * (k + 1), K, V, dev)
    _check(lib().verify_accept_x(_ptr(x), B, k, K, _ptr(W.base), _ptr(W.refine), _ptr(W.scales), V, group,
                                 _ptr(draft), _ptr(out["target"]), _ptr(out["n_emitted"]),
                                 _ptr(out["emitted"]), _ptr(out.get("y")), _ptr(length), _ptr(next_token),
                                 _ptr(ws), ws.numel(), _stream(dev)), what)
    return out


def verify_accept_x_static(x, B: int, k: int, W, draft, group: int = 128, want_y: bool = False, out=None,
                           length=None, next_token=None):
    """verify_accept_x on the library's own per-device scratch (no workspace)."""
    what = "verify_accept_x_static"
    _dev(x, torch.float32, what, "x")
    _dev(draft, torch.int32, what, "draft")
    W = _tiled(W, what, 2)
    K = x.shape[1]
    V = W.rows
    dev = x.device
    if out is None:
        out = _accept_out(B, k, V, dev, want_y)
    _check(lib().verify_accept_x_static(_ptr(x), B, k, K, _ptr(W.base), _ptr(W.refine), _ptr(W.scales), V,
                                        group, _ptr(draft), _ptr(out["target"]), _ptr(out["n_emitted"]),
                                        _ptr(out["emitted"]), _ptr(out.get("y")), _ptr(length),
                                        _ptr(next_token), _stream(dev)), what)
    return out


class NestKV:
    """A nested KV cache in device memory (layouts in include/nestspec.h)."""

    def __init__(self, k_base, k_refine, k_scale, v_base, v_refine, v_scale, n_kv_heads,
                 capacity, head_dim, block):
        self.k_base, self.k_refine, self.k_scale = k_base, k_refine, k_scale
        self.v_base, self.v_refine, self.v_scale = v_base, v_refine, v_scale
        self.n_kv_heads, self.capacity, self.head_dim, self.block = (
            int(n_kv_heads), int(capacity), int(head_dim), int(block))

    def struct(self) -> _KV:
        return _KV(self.k_base.data_ptr(), self.k_refine.data_ptr() if self.k_refine is not None else 0,
                   self.k_scale.data_ptr(), self.v_base.data_ptr(),
                   self.v_refine.data_ptr() if self.v_refine is not None else 0,
                   self.v_scale.data_ptr(), self.n_kv_heads, self.head_dim, self.capacity, self.block)


def kv_nest_pack(k: torch.Tensor, v: torch.Tensor, block: int = 128) -> NestKV:
    """fp32 K and V [Hkv][capacity][d] -> NestKV."""
    what = "kv_nest_pack"
    _dev(k, torch.float32, what, "k")
    _dev(v, torch.float32, what, "v")
    Hkv, cap, d = k.shape
    dev = k.device
    n = Hkv * cap * d // 2
    planes = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(4)]
    ks = torch.empty((Hkv, cap // block), dtype=torch.float32, device=dev)
    vs = torch.empty((Hkv, cap // block), dtype=torch.float32, device=dev)
    _check(lib().kv_nest_pack(_ptr(k), _ptr(v), Hkv, cap, d, block, _ptr(planes[0]),
                              _ptr(planes[1]), _ptr(ks), _ptr(planes[2]), _ptr(planes[3]),
                              _ptr(vs), _stream(dev)), what)
    return NestKV(planes[0], planes[1], ks, planes[2], planes[3], vs, Hkv, cap, d, block)


def kv_shadow(kv: NestKV):
    """fp32 shadows (K, V) of the two most recent blocks, for kv_nest_append."""
    n = lib().kv_nest_shadow_floats(kv.n_kv_heads, kv.head_dim, kv.block)
    dev = kv.k_base.device
    return (torch.zeros(n, dtype=torch.float32, device=dev), torch.zeros(n, dtype=torch.float32, device=dev))


def kv_nest_shadow_fill(kv: NestKV, k: torch.Tensor, v: torch.Tensor, ctx_len: int, shadow):
    """Carry the open block's fp32 tokens of k, v [Hkv][src_len][d] into the shadows."""
    what = "kv_nest_shadow_fill"
    _dev(k, torch.float32, what, "k")
    _dev(v, torch.float32, what, "v")
    s = kv.struct()
    _check(lib().kv_nest_shadow_fill(ctypes.byref(s), _ptr(k), _ptr(v), k.shape[1], int(ctx_len),
                                     _ptr(shadow[0]), _ptr(shadow[1]), _stream(k.device)), what)


def kv_nest_append(kv: NestKV, shadow, k_new: torch.Tensor, v_new: torch.Tensor, pos: int, pos_dev=None):
    """Write fp32 k_new, v_new [Hkv][n][d] at positions pos.. (pos plus the
    device int32 pos_dev when given) and quantize the touched blocks again."""
    what = "kv_nest_append"
    _dev(k_new, torch.float32, what, "k_new")
    _dev(v_new, torch.float32, what, "v_new")
    if pos_dev is not None:
        _dev(pos_dev, torch.int32, what, "pos_dev")
    s = kv.struct()
    _check(lib().kv_nest_append(ctypes.byref(s), _ptr(shadow[0]), _ptr(shadow[1]), _ptr(k_new), _ptr(v_new),
                                _ptr(pos_dev), int(pos), k_new.shape[1], _stream(k_new.device)), what)


def kv_nest_attend(q: torch.Tensor, kv: NestKV, ctx_len: int, view: int, out=None, ws=None, ctx_dev=None):
    """q: bf16 [nq][Hq][d] (torch.bfloat16, or its bit patterns as int16/uint16).
    The visible length is ctx_len, plus the device int32 ctx_dev when given.
    Returns fp32 [nq][Hq][d]."""
    what = "kv_nest_attend"
    if not isinstance(q, torch.Tensor) or not q.is_cuda or not q.is_contiguous():
        raise NestError(f"{what}: q must be a contiguous CUDA tensor")
    if q.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise NestError(f"{what}: q must hold bf16 bit patterns")
    if ctx_dev is not None:
        _dev(ctx_dev, torch.int32, what, "ctx_dev")
    nq, Hq, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((nq, Hq, d), dtype=torch.float32, device=dev)
    plan_len = kv.capacity if ctx_dev is not None else int(ctx_len)
    wsn = lib().kv_nest_attend_workspace_size(nq, Hq, kv.n_kv_heads, d, plan_len)
    if ws is None or ws.numel() < wsn:
        ws = workspace(max(wsn, 256), dev, "attend")
    s = kv.struct()
    _check(lib().kv_nest_attend(_ptr(q), nq, Hq, ctypes.byref(s), _ptr(ctx_dev), int(ctx_len), int(view),
                                _ptr(out), _ptr(ws), ws.numel(), _stream(dev)), what)
    return out


def kv_nest_attend_exact(q: torch.Tensor, kv: NestKV, shadow, ctx_len: int, view: int, out=None, ws=None,
                         ctx_dev=None):
    """The nq queries of one verify pass, each exactly as a one-query call at
    its own position (after kv_nest_append of the nq tokens). q: bf16 bits
    [nq][Hq][d]. Returns fp32 [nq][Hq][d]."""
    what = "kv_nest_attend_exact"
    if not isinstance(q, torch.Tensor) or not q.is_cuda or not q.is_contiguous():
        raise NestError(f"{what}: q must be a contiguous CUDA tensor")
    if q.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise NestError(f"{what}: q must hold bf16 bit patterns")
    if ctx_dev is not None:
        _dev(ctx_dev, torch.int32, what, "ctx_dev")
    nq, Hq, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((nq, Hq, d), dtype=torch.float32, device=dev)
    plan_len = kv.capacity if ctx_dev is not None else int(ctx_len)
    wsn = lib().kv_nest_attend_exact_workspace_size(nq, Hq, kv.n_kv_heads, d, plan_len)
    if ws is None or ws.numel() < wsn:
        ws = workspace(max(wsn, 256), dev, "attend")
    s = kv.struct()
    _check(lib().kv_nest_attend_exact(_ptr(q), nq, Hq, ctypes.byref(s), _ptr(shadow[0]), _ptr(shadow[1]),
                                      _ptr(ctx_dev), int(ctx_len), int(view), _ptr(out), _ptr(ws), ws.numel(),
                                      _stream(dev)), what)
    return out


def kv_nest_append_attend_exact(q: torch.Tensor, kv: NestKV, shadow, k_new: torch.Tensor, v_new: torch.Tensor,
                                pos: int, view: int, out=None, ws=None, pos_dev=None):
    """kv_nest_append of the n new tokens k_new, v_new [Hkv][n][d] at
    positions pos.. (plus the device int32 pos_dev when given), then
    kv_nest_attend_exact of q [n][Hq][d] (bf16 bits) at length pos + n, in
    one call with one launch fewer. Returns fp32 [n][Hq][d]."""
    what = "kv_nest_append_attend_exact"
    if not isinstance(q, torch.Tensor) or not q.is_cuda or not q.is_contiguous():
        raise NestError(f"{what}: q must be a contiguous CUDA tensor")
    if q.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise NestError(f"{what}: q must hold bf16 bit patterns")
    _dev(k_new, torch.float32, what, "k_new")
    _dev(v_new, torch.float32, what, "v_new")
    if pos_dev is not None:
        _dev(pos_dev, torch.int32, what, "pos_dev")
    n, Hq, d = q.shape
    dev = q.device
    if out is None:
        out = torch.empty((n, Hq, d), dtype=torch.float32, device=dev)
    plan_len = kv.capacity if pos_dev is not None else int(pos) + n
    wsn = lib().kv_nest_attend_exact_workspace_size(n, Hq, kv.n_kv_heads, d, plan_len)
    if ws is None or ws.numel() < wsn:
        ws = workspace(max(wsn, 256), dev, "attend")
    s = kv.struct()
    _check(lib().kv_nest_append_attend_exact(_ptr(q), n, Hq, ctypes.byref(s), _ptr(shadow[0]), _ptr(shadow[1]),
                                             _ptr(k_new), _ptr(v_new), _ptr(pos_dev), int(pos), int(view),
                                             _ptr(out), _ptr(ws), ws.numel(), _stream(dev)), what)
    return out


# ---------------------------------------------------------------------------
# choosing k (host functions of the library; no GPU involved)
# ---------------------------------------------------------------------------

def expected_tokens(alpha: float, k: int) -> float:
    """Eq. (1)."""
    return lib().nest_expected_tokens(float(alpha), int(k))


def token_time(alpha: float, k: int, t_draft: float, t_pass: float) -> float:
    """Eq. (2)."""
    return lib().nest_token_time(float(alpha), int(k), float(t_draft), float(t_pass))


def sample(y, temperature: float, u, tokens=None, ws=None):
    """One id per row of the fp32 logits y [M][V] from softmax(y / T), drawn
    by inverse CDF with the fp32 uniforms u [M]. Returns int32 [M]."""
    what = "nest_sample"
    _dev(y, torch.float32, what, "y")
    _dev(u, torch.float32, what, "u")
    M, V = y.shape
    if u.numel() != M:
        raise NestError(f"{what}: u needs {M} values")
    dev = y.device
    if tokens is None:
        tokens = torch.empty(M, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(lib().nest_sample_workspace_size(M, V), dev, "sample")
    _check(lib().nest_sample(_ptr(y), M, V, float(temperature), _ptr(u), _ptr(tokens), _ptr(ws), ws.numel(),
                             _stream(dev)), what)
    return tokens


def verify_sample(yt, yd, draft, temperature: float, u_acc, u_fin, out=None, ws=None):
    """Accept test and last draw of B speculative-sampling rounds.
    yt fp32 [B][k+1][V], yd fp32 [B][k][V] (or None when k == 0), draft
    int32 [B][k], u_acc fp32 [B][k], u_fin fp32 [B]. Returns a dict of device
    tensors n_emitted [B] and emitted [B][k+1]."""
    what = "verify_sample"
    _dev(yt, torch.float32, what, "yt")
    B, k1, V = yt.shape
    k = k1 - 1
    if k > 0:
        _dev(yd, torch.float32, what, "yd")
        _dev(draft, torch.int32, what, "draft")
        _dev(u_acc, torch.float32, what, "u_acc")
        if tuple(yd.shape) != (B, k, V) or draft.numel() != B * k or u_acc.numel() != B * k:
            raise NestError(f"{what}: yd, draft and u_acc must hold [B][k] rows")
    _dev(u_fin, torch.float32, what, "u_fin")
    if u_fin.numel() != B:
        raise NestError(f"{what}: u_fin needs {B} values")
    dev = yt.device
    if out is None:
        out = {"n_emitted": torch.empty(B, dtype=torch.int32, device=dev),
               "emitted": torch.empty((B, k1), dtype=torch.int32, device=dev)}
    if ws is None:
        ws = workspace(lib().verify_sample_workspace_size(B, k, V), dev, "verify_sample")
    _check(lib().verify_sample(_ptr(yt), _ptr(yd) if k else None, B, k, V, float(temperature),
                               _ptr(draft) if k else None, _ptr(u_acc) if k else None, _ptr(u_fin),
                               _ptr(out["n_emitted"]), _ptr(out["emitted"]), _ptr(ws), ws.numel(),
                               _stream(dev)), what)
    return out


def embed(table, tokens, out=None):
    """out [M][H] = table[tokens] (fp32 table [V][H], int32 tokens [M])."""
    what = "nest_embed"
    _dev(table, torch.float32, what, "table")
    _dev(tokens, torch.int32, what, "tokens")
    V, H = table.shape
    M = tokens.numel()
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32, device=table.device)
    _check(lib().nest_embed(_ptr(table), V, H, _ptr(tokens), M, _ptr(out), _stream(table.device)), what)
    return out


def add_rmsnorm(x, y, gamma, eps: float, out=None):
    """x += y (when y is given, in place), then RMSNorm of x with gamma."""
    what = "nest_add_rmsnorm"
    _dev(x, torch.float32, what, "x")
    _dev(gamma, torch.float32, what, "gamma")
    if y is not None:
        _dev(y, torch.float32, what, "y")
    M, H = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib().nest_add_rmsnorm(_ptr(x), _ptr(y), _ptr(gamma), M, H, float(eps), _ptr(out),
                                  _stream(x.device)), what)
    return out


def rope_split(qkv, pos0: int, n_q_heads: int, n_kv_heads: int, head_dim: int, theta: float,
               token_major: bool = False, out=None, pos_dev=None):
    """Rotary embedding + q/k/v split of qkv [M][(Hq+2Hkv)d] at positions
    pos0 + m (plus the device int32 pos_dev when given): (q bf16 bits
    [M][Hq][d] as int16, k, v fp32 [Hkv][M][d] or [M][Hkv][d])."""
    what = "nest_rope_split"
    _dev(qkv, torch.float32, what, "qkv")
    M = qkv.shape[0]
    dev = qkv.device
    if out is None:
        kv_shape = (M, n_kv_heads, head_dim) if token_major else (n_kv_heads, M, head_dim)
        out = (torch.empty((M, n_q_heads, head_dim), dtype=torch.int16, device=dev),
               torch.empty(kv_shape, dtype=torch.float32, device=dev),
               torch.empty(kv_shape, dtype=torch.float32, device=dev))
    q, k, v = out
    _check(lib().nest_rope_split(_ptr(qkv), M, _ptr(pos_dev), int(pos0), n_q_heads, n_kv_heads, head_dim,
                                 float(theta), 1 if token_major else 0, _ptr(q), _ptr(k), _ptr(v),
                                 _stream(dev)), what)
    return q, k, v


def swiglu(gate_up, out=None):
    """silu(gate) * up for gate_up [M][2I]."""
    what = "nest_swiglu"
    _dev(gate_up, torch.float32, what, "gate_up")
    M, I2 = gate_up.shape
    if out is None:
        out = torch.empty((M, I2 // 2), dtype=torch.float32, device=gate_up.device)
    _check(lib().nest_swiglu(_ptr(gate_up), M, I2 // 2, _ptr(out), _stream(gate_up.device)), what)
    return out


def choose_k(alpha: float, t_draft: float, t_pass):
    """(k, time per token) minimising Eq. (2) over k = 0 .. len(t_pass)-1."""
    import numpy as np

    tp = np.ascontiguousarray(t_pass, dtype=np.float64)
    out = ctypes.c_double(0.0)
    k = lib().nest_choose_k(float(alpha), float(t_draft), tp.ctypes.data_as(ctypes.c_void_p), tp.size - 1,
                            ctypes.byref(out))
    if k < 0:
        _check(1, "nest_choose_k")
    return int(k), out.value


class AlphaEstimate:
    """Running acceptance rate (nest_alpha)."""

    def __init__(self, decay: float = 1.0, prior_accepted: float = 1.0, prior_rejected: float = 1.0):
        self._st = _Alpha()
        lib().nest_alpha_init(ctypes.byref(self._st), float(decay), float(prior_accepted),
                              float(prior_rejected))

    def update(self, accepted: int, k: int) -> float:
        lib().nest_alpha_update(ctypes.byref(self._st), int(accepted), int(k))
        return self.value

    @property
    def value(self) -> float:
        return lib().nest_alpha_value(ctypes.byref(self._st))
