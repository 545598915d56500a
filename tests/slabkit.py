"""Hand-built expert slabs, written directly from the slab layout description.

Layout (per matrix with R rows and K columns): R*K/2 code bytes, row-major, byte b
of a row holding column 2b in bits 0-3 and column 2b+1 in bits 4-7; then R*(K/32)
4-byte records (fp16 scale, fp16 min) row-major over (row, 32-column block).
Slab = W1 (gate, [I x H]) | W3 (up, [I x H]) | W2 (down, [H x I]).
"""
import numpy as np


def f16(v):
    """fp16 bit pattern of a value (numpy rounds to nearest even)."""
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def pack_matrix(q, scale_bits, min_bits):
    q = np.asarray(q, dtype=np.int64)
    R, K = q.shape
    assert K % 32 == 0 and q.min() >= 0 and q.max() <= 15
    sc = np.broadcast_to(np.asarray(scale_bits, dtype=np.uint16), (R, K // 32))
    mn = np.broadcast_to(np.asarray(min_bits, dtype=np.uint16), (R, K // 32))
    codes = bytearray(R * K // 2)
    for r in range(R):
        for b in range(K // 2):
            codes[r * (K // 2) + b] = int(q[r, 2 * b]) | (int(q[r, 2 * b + 1]) << 4)
    params = bytearray(R * (K // 32) * 4)
    for r in range(R):
        for j in range(K // 32):
            o = (r * (K // 32) + j) * 4
            s, m = int(sc[r, j]), int(mn[r, j])
            params[o:o + 4] = bytes([s & 0xFF, s >> 8, m & 0xFF, m >> 8])
    return bytes(codes) + bytes(params)


def build_slab(H, I, w1, w3, w2):
    """Each of w1/w3/w2 is a (q, scale_bits, min_bits) triple."""
    blob = pack_matrix(*w1) + pack_matrix(*w3) + pack_matrix(*w2)
    assert len(blob) == int(1.875 * H * I)
    return np.frombuffer(blob, dtype=np.uint8).copy()


def constant_matrix(R, K, code, scale):
    """Every code `code`, every block scale `scale`, min = -8*scale: W = scale*(code-8)."""
    q = np.full((R, K), code)
    return (q, f16(scale), f16(-8.0 * scale))


def dequant_expected(q, scale_bits, min_bits):
    """Expected dequantised matrix, from the layout's value rule scale*q + min."""
    q = np.asarray(q, dtype=np.float64)
    R, K = q.shape
    sc = np.broadcast_to(np.asarray(scale_bits, np.uint16), (R, K // 32)).view(np.float16).astype(np.float64)
    mn = np.broadcast_to(np.asarray(min_bits, np.uint16), (R, K // 32)).view(np.float16).astype(np.float64)
    return np.repeat(sc, 32, axis=1) * q + np.repeat(mn, 32, axis=1)
