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
