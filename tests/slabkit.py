"""Hand-built expert slabs, written directly from the slab layout description.

Layout: a row of a matrix with K columns is K/2 code bytes (byte b holds column 2b
in bits 0-3 and column 2b+1 in bits 4-7) followed by K/32 4-byte records (fp16
scale, fp16 min), one per 32-column block, zero-padded to a multiple of 16 bytes.
Slab = for each r < I the pair (W1 row r, W3 row r) (gate and up, [I x H]), then
the H rows of W2 (down, [H x I]).
"""
import numpy as np


def f16(v):
    """fp16 bit pattern of a value (numpy rounds to nearest even)."""
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def row_bytes(K):
    """Codes and records of a K-column row, zero-padded to a multiple of 16 bytes."""
    return (K // 2 + (K // 32) * 4 + 15) // 16 * 16


def pack_rows(q, scale_bits, min_bits):
    """The rows of one matrix, each as its own bytes (codes, then records)."""
    q = np.asarray(q, dtype=np.int64)
    R, K = q.shape
    assert K % 32 == 0 and q.min() >= 0 and q.max() <= 15
    sc = np.broadcast_to(np.asarray(scale_bits, dtype=np.uint16), (R, K // 32))
    mn = np.broadcast_to(np.asarray(min_bits, dtype=np.uint16), (R, K // 32))
    rows = []
    for r in range(R):
        row = bytearray(row_bytes(K))
        for b in range(K // 2):
            row[b] = int(q[r, 2 * b]) | (int(q[r, 2 * b + 1]) << 4)
        for j in range(K // 32):
            o = K // 2 + 4 * j
            s, m = int(sc[r, j]), int(mn[r, j])
            row[o:o + 4] = bytes([s & 0xFF, s >> 8, m & 0xFF, m >> 8])
        rows.append(bytes(row))
    return rows


def build_slab(H, I, w1, w3, w2):
    """Each of w1/w3/w2 is a (q, scale_bits, min_bits) triple."""
    r1, r3, r2 = pack_rows(*w1), pack_rows(*w3), pack_rows(*w2)
    assert len(r1) == len(r3) == I and len(r2) == H
    blob = b"".join(a + b for a, b in zip(r1, r3)) + b"".join(r2)
    assert len(blob) == 2 * I * row_bytes(H) + H * row_bytes(I)
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


def row_view(slab, H, I, which):
    """[rows, row bytes] view of matrix `which` (0 = W1, 1 = W3, 2 = W2) of a slab."""
    slab = np.asarray(slab, dtype=np.uint8)
    gate_row, down_row = row_bytes(H), row_bytes(I)
    if which < 2:
        pairs = slab[:I * 2 * gate_row].reshape(I, 2 * gate_row)
        return pairs[:, which * gate_row:(which + 1) * gate_row]
    return slab[I * 2 * gate_row:].reshape(H, down_row)


def records_of(slab, H, I, which):
    """(scale, min) fp16 bit patterns of every block of a matrix: [rows, K/32, 2] uint16."""
    K = H if which < 2 else I
    rows = np.ascontiguousarray(row_view(slab, H, I, which)[:, K // 2:K // 2 + (K // 32) * 4])
    return rows.view(np.uint16).reshape(rows.shape[0], K // 32, 2)
