"""Independent decoders of the documented storage formats, for the tests.

They are written from the format definitions in include/nestspec.h
(nibble order, plane shapes, the K and V cache layouts). They share nothing
with the oracle or the HIP library, so a layout mistake in either one shows
up as a mismatch against these.
"""
import numpy as np


def decode_plane(plane: np.ndarray, n_elems: int | None = None) -> np.ndarray:
    """uint8 plane -> int8 codes. Element 2j is the low nibble of byte j and
    element 2j+1 the high nibble, both 4-bit two's complement."""
    b = np.asarray(plane, dtype=np.uint8).reshape(-1)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    out = np.empty(b.size * 2, dtype=np.int16)
    out[0::2] = lo
    out[1::2] = hi
    out = np.where(out >= 8, out - 16, out).astype(np.int8)
    return out if n_elems is None else out[:n_elems]


def decode_matrix(plane: np.ndarray, rows: int, cols: int) -> np.ndarray:
    return decode_plane(plane, rows * cols).reshape(rows, cols)


def decode_k_cache(plane, n_kv_heads, capacity, head_dim) -> np.ndarray:
    """K cache plane (token-major) -> codes [Hkv][capacity][d]."""
    return decode_plane(plane, n_kv_heads * capacity * head_dim).reshape(
        n_kv_heads, capacity, head_dim)


def decode_v_cache(plane, n_kv_heads, capacity, head_dim, block) -> np.ndarray:
    """V cache plane (dim-major inside each block) -> codes [Hkv][capacity][d]."""
    c = decode_plane(plane, n_kv_heads * capacity * head_dim).reshape(
        n_kv_heads, capacity // block, head_dim, block)
    return c.transpose(0, 1, 3, 2).reshape(n_kv_heads, capacity, head_dim)


def block_scales_per_token(scales, capacity, block) -> np.ndarray:
    """[Hkv][capacity/block] -> [Hkv][capacity] (each token's block scale)."""
    return np.repeat(np.asarray(scales, dtype=np.float64), block, axis=1)[:, :capacity]


def tile_plane(plane: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Storage plane uint8 [rows][cols/2] -> the tile layout of nestspec.h:
    rows padded with zeros to T*16, then per (tile t, group g) the kilobyte
    [k-quarter q][row r][16 bytes] = bytes 64g + 16q .. +15 of row 16t + r."""
    T, G = -(-rows // 16), cols // 128
    p = np.zeros((T * 16, cols // 2), np.uint8)
    p[:rows] = np.asarray(plane, np.uint8).reshape(rows, cols // 2)
    return p.reshape(T, 16, G, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)


def tile_scales(scales: np.ndarray, rows: int, G: int) -> np.ndarray:
    """Storage scales fp32 [rows][G] -> the tile layout: rows padded to
    T*16 and groups to Gq*4 with zeros, then [t][quad u][row r][i]."""
    T, Gq = -(-rows // 16), -(-G // 4)
    s = np.zeros((T * 16, Gq * 4), np.float32)
    s[:rows, :G] = np.asarray(scales, np.float32).reshape(rows, G)
    return s.reshape(T, 16, Gq, 4).transpose(0, 2, 1, 3).reshape(-1)
