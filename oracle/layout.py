"""Tiled byte layout of packed weights, written from its prose spec with numpy
reshapes and transposes (test infrastructure only).

This layout is the library's own design, not the pages' (parity unpinned by
the pages; pinned by the tests' bijection, size and hand-derived offset
checks).  The prose spec it follows:

Common
  Rows are padded to Np = 16*ceil(N/16) and K to Kp = 256*ceil(K/256); padded
  codes, scales and mins are zero.  Row-group r covers rows 16r..16r+15,
  super-block j covers k = 256j..256j+255.  Tile (r, j) starts at byte
  (r*(Kp/256) + j) * T, T being the tile size, so a row-group's tiles are
  contiguous.  In a 1024-byte chunk, "lane" l = 16g + rho (0 <= l < 64) owns
  bytes 16l..16l+15, row 16r + rho, and K quarter g.

int8 b32 tile (T = 4352 = 4*1024 + 256)
  Chunk s (0..3), lane (g, rho):
    bytes 0..7  = codes[n, 256j + 64s + 8g + i],        i = 0..7
    bytes 8..15 = codes[n, 256j + 64s + 32 + 8g + i],   i = 0..7
  so bytes 0..7 of all lanes cover block 8j+2s and bytes 8..15 block 8j+2s+1.
  Bytes 4096..4351: row rho's 8 scales (blocks 8j..8j+7, fp16 little endian)
  at 4096 + 16*rho.

int4 g64 tile (T = 2304 = 2*1024 + 256)
  Chunk s (0..1), lane (g, rho):
    bytes 0..7  = codes of group 4j+2s,   in-group offsets 16g..16g+15
    bytes 8..15 = codes of group 4j+2s+1, in-group offsets 16g..16g+15
  as two little-endian uint32 words per 8 bytes, each word holding 8
  consecutive codes k0..k0+7 with nibble p (bits 4p..4p+3) holding code
  k0 + PERM4[p], PERM4 = (0, 2, 4, 6, 1, 3, 5, 7).
  Bytes 2048..2303: row rho's 16 bytes at 2048 + 16*rho = 4 fp16 scales
  (groups 4j..4j+3) then 4 fp16 mins (same groups).

fp16 tile (T = 8192 = 8*1024)
  Chunk s (0..7), lane (g, rho): bytes 0..15 = w16[n, 256j + 32s + 8g + i],
  i = 0..7 (fp16 little endian), so chunk s holds the 32-wide block 8j+s.
"""
from __future__ import annotations

import numpy as np

TILE_ROWS = 16
SUPER_K = 256
TILE_BYTES_INT8 = 4352
TILE_BYTES_INT4 = 2304
TILE_BYTES_FP16 = 8192
TILE_BYTES = {"int8_b32": TILE_BYTES_INT8, "int4_g64": TILE_BYTES_INT4, "fp16": TILE_BYTES_FP16}
PERM4 = (0, 2, 4, 6, 1, 3, 5, 7)


def padded(n: int, k: int):
    np_ = -(-n // TILE_ROWS) * TILE_ROWS
    kp = -(-k // SUPER_K) * SUPER_K
    return np_, kp


def packed_bytes(fmt: str, n: int, k: int) -> int:
    np_, kp = padded(n, k)
    return (np_ // TILE_ROWS) * (kp // SUPER_K) * TILE_BYTES[fmt]


def _pad(a: np.ndarray, rows: int, cols: int) -> np.ndarray:
    out = np.zeros((rows, cols), a.dtype)
    out[: a.shape[0], : a.shape[1]] = a
    return out


def tile_int8_b32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(int8 [N, K], fp16 [N, K/32]) -> uint8 blob."""
    n, k = codes.shape
    np_, kp = padded(n, k)
    R, J = np_ // 16, kp // 256
    c = _pad(codes.astype(np.int8), np_, kp)
    s = _pad(scales.astype(np.float16), np_, kp // 32)
    # k = 256 j + 64 s + 32 h + 8 g + i ;  n = 16 r + rho
    c = c.reshape(R, 16, J, 4, 2, 4, 8)           # r rho j s h g i
    c = c.transpose(0, 2, 3, 5, 1, 4, 6)          # r j s g rho h i
    c = c.reshape(R, J, 4096).view(np.uint8)
    sc = s.reshape(R, 16, J, 8).transpose(0, 2, 1, 3)   # r j rho beta
    sc = np.ascontiguousarray(sc).view(np.uint8).reshape(R, J, 256)
    return np.concatenate([c, sc], axis=2).reshape(-1)


def untile_int8_b32(blob: np.ndarray, n: int, k: int):
    """Inverse of ``tile_int8_b32`` (drops the padding)."""
    np_, kp = padded(n, k)
    R, J = np_ // 16, kp // 256
    t = blob.reshape(R, J, TILE_BYTES_INT8)
    c = t[:, :, :4096].copy().view(np.int8).reshape(R, J, 4, 4, 16, 2, 8)   # r j s g rho h i
    c = c.transpose(0, 4, 1, 2, 5, 3, 6).reshape(np_, kp)                  # r rho j s h g i
    sc = t[:, :, 4096:].copy().view(np.float16).reshape(R, J, 16, 8)       # r j rho beta
    sc = sc.transpose(0, 2, 1, 3).reshape(np_, kp // 32)
    return c[:n, :k].copy(), sc[:n, : k // 32].copy()


def _words_from_codes(q: np.ndarray) -> np.ndarray:
    """[..., 8] codes (consecutive k) -> [...] uint32 with nibble p = code PERM4[p]."""
    q = q.astype(np.uint32)
    w = np.zeros(q.shape[:-1], np.uint32)
    for p in range(8):
        w |= q[..., PERM4[p]] << np.uint32(4 * p)
    return w


def _codes_from_words(w: np.ndarray) -> np.ndarray:
    out = np.empty(w.shape + (8,), np.uint8)
    for p in range(8):
        out[..., PERM4[p]] = (w >> np.uint32(4 * p)) & np.uint32(0xF)
    return out


def tile_int4_g64(codes: np.ndarray, scales: np.ndarray, mins: np.ndarray) -> np.ndarray:
    """(uint8 codes [N, K] in 0..15, fp16 scales/mins [N, K/64]) -> uint8 blob."""
    n, k = codes.shape
    np_, kp = padded(n, k)
    R, J = np_ // 16, kp // 256
    q = _pad(codes.astype(np.uint8), np_, kp)
    s = _pad(scales.astype(np.float16), np_, kp // 64)
    m = _pad(mins.astype(np.float16), np_, kp // 64)
    # k = 256 j + 128 s + 64 h + 16 g + 8 w + c
    q = q.reshape(R, 16, J, 2, 2, 4, 2, 8)         # r rho j s h g w c
    q = q.transpose(0, 2, 3, 5, 1, 4, 6, 7)        # r j s g rho h w c
    words = _words_from_codes(q)                   # r j s g rho h w
    cb = np.ascontiguousarray(words).astype("<u4").view(np.uint8).reshape(R, J, 2048)
    sc = s.reshape(R, 16, J, 4).transpose(0, 2, 1, 3)   # r j rho grp
    mn = m.reshape(R, 16, J, 4).transpose(0, 2, 1, 3)
    meta = np.ascontiguousarray(np.concatenate([sc, mn], axis=3)).view(np.uint8).reshape(R, J, 256)
    return np.concatenate([cb, meta], axis=2).reshape(-1)


def untile_int4_g64(blob: np.ndarray, n: int, k: int):
    """Inverse of ``tile_int4_g64`` (drops the padding)."""
    np_, kp = padded(n, k)
    R, J = np_ // 16, kp // 256
    t = blob.reshape(R, J, TILE_BYTES_INT4)
    words = t[:, :, :2048].copy().view("<u4").reshape(R, J, 2, 4, 16, 2, 2)   # r j s g rho h w
    q = _codes_from_words(words)                                             # + c
    q = q.transpose(0, 4, 1, 2, 5, 3, 6, 7).reshape(np_, kp)                 # r rho j s h g w c
    meta = t[:, :, 2048:].copy().view(np.float16).reshape(R, J, 16, 8)
    sc = meta[..., :4].transpose(0, 2, 1, 3).reshape(np_, kp // 64)
    mn = meta[..., 4:].transpose(0, 2, 1, 3).reshape(np_, kp // 64)
    return q[:n, :k].copy(), sc[:n, : k // 64].copy(), mn[:n, : k // 64].copy()


def tile_fp16(w16: np.ndarray) -> np.ndarray:
    """fp16 [N, K] -> uint8 blob."""
    n, k = w16.shape
    np_, kp = padded(n, k)
    R, J = np_ // 16, kp // 256
    w = _pad(w16.astype(np.float16), np_, kp)
    # k = 256 j + 32 s + 8 g + i ;  n = 16 r + rho
    w = w.reshape(R, 16, J, 8, 4, 8)             # r rho j s g i
    w = w.transpose(0, 2, 3, 4, 1, 5)            # r j s g rho i
    return np.ascontiguousarray(w).astype("<f2").view(np.uint8).reshape(-1)


def untile_fp16(blob: np.ndarray, n: int, k: int):
    """Inverse of ``tile_fp16`` (drops the padding); returns (w16,)."""
    np_, kp = padded(n, k)
    R, J = np_ // 16, kp // 256
    w = blob.reshape(R, J, TILE_BYTES_FP16).copy().view("<f2").reshape(R, J, 8, 4, 16, 8)  # r j s g rho i
    w = w.transpose(0, 4, 1, 2, 3, 5).reshape(np_, kp)                                    # r rho j s g i
    return (w[:n, :k].astype(np.float16).copy(),)


def row_group_slice(fmt: str, n: int, k: int, r: int) -> slice:
    """Byte range of row-group r (rows 16r..16r+15) inside a blob."""
    _, kp = padded(n, k)
    span = (kp // SUPER_K) * TILE_BYTES[fmt]
    return slice(r * span, (r + 1) * span)
