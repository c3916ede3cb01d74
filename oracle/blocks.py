"""GGUF block decoding (Q8_0, Q4_0) and f32 tensors, written from the definitions.

Synsema "Local inference and architectures", section "Choose the engine": the
weights stay block-quantized and the engine multiplies them in f32.  The block
layouts themselves are not printed on the pages; this follows GGUF's public
layout (ggml type ids F32 = 0, Q4_0 = 2, Q8_0 = 8):

  Q8_0 block (34 B): fp16 scale d, int8 q[32];            w[j] = d * q[j]
  Q4_0 block (18 B): fp16 scale d, uint8 b[16];           w[j]      = d * ((b[j] & 15) - 8)
                                                          w[j + 16] = d * ((b[j] >> 4) - 8)

Blocks run along the input dimension of each output row; a row holds
ceil(cols/32) blocks and only its first ``cols`` values are logical.
The product d*q is exact in f32 (11 + 8 significant bits), so the decode is
exact and the result is returned as float32.
"""
import numpy as np

T_F32 = 0
T_Q4_0 = 2
T_Q8_0 = 8


def _nblk(cols):
    return (cols + 31) // 32


def _f16_to_f32(u16):
    """IEEE binary16 bits -> float32 value, written out (sign, exponent, mantissa)."""
    u = u16.astype(np.uint32)
    sign = np.where(u >> 15, -1.0, 1.0)
    e = (u >> 10) & 0x1F
    m = (u & 0x3FF).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 1024.0, e.astype(np.int64) - 15)
    sub = sign * np.ldexp(m / 1024.0, -14)
    special = np.where(m == 0, sign * np.inf, np.nan)
    out = np.where(e == 0, sub, np.where(e == 31, special, normal))
    return out.astype(np.float32)


def dequant_q8_0(raw, rows, cols):
    """Decode Q8_0 bytes into f32 [rows][cols]."""
    nb = _nblk(cols)
    b = np.frombuffer(np.asarray(raw, dtype=np.uint8).tobytes(), dtype=np.uint8)
    if b.size != rows * nb * 34:
        raise ValueError(f"Q8_0: expected {rows * nb * 34} bytes, got {b.size}")
    blk = b.reshape(rows, nb, 34)
    d = _f16_to_f32(blk[:, :, 0].astype(np.uint16) | (blk[:, :, 1].astype(np.uint16) << 8))
    q = blk[:, :, 2:].view(np.int8).astype(np.float32)
    w = d[:, :, None] * q
    return np.ascontiguousarray(w.reshape(rows, nb * 32)[:, :cols])


def dequant_q4_0(raw, rows, cols):
    """Decode Q4_0 bytes into f32 [rows][cols]."""
    nb = _nblk(cols)
    b = np.frombuffer(np.asarray(raw, dtype=np.uint8).tobytes(), dtype=np.uint8)
    if b.size != rows * nb * 18:
        raise ValueError(f"Q4_0: expected {rows * nb * 18} bytes, got {b.size}")
    blk = b.reshape(rows, nb, 18)
    d = _f16_to_f32(blk[:, :, 0].astype(np.uint16) | (blk[:, :, 1].astype(np.uint16) << 8))
    payload = blk[:, :, 2:]
    lo = (payload & 0x0F).astype(np.float32) - 8.0
    hi = (payload >> 4).astype(np.float32) - 8.0
    n = np.concatenate([lo, hi], axis=2)  # elements 0..15 from low nibbles, 16..31 from high
    w = d[:, :, None] * n
    return np.ascontiguousarray(w.reshape(rows, nb * 32)[:, :cols])


def dequant_f32(raw, rows, cols):
    b = np.frombuffer(np.asarray(raw, dtype=np.uint8).tobytes(), dtype="<f4")
    if b.size != rows * cols:
        raise ValueError(f"F32: expected {rows * cols * 4} bytes, got {b.size * 4}")
    return b.reshape(rows, cols).copy()


def dequant(ttype, raw, rows, cols):
    """Decode any supported tensor into f32 [rows][cols]."""
    if ttype == T_Q8_0:
        return dequant_q8_0(raw, rows, cols)
    if ttype == T_Q4_0:
        return dequant_q4_0(raw, rows, cols)
    if ttype == T_F32:
        return dequant_f32(raw, rows, cols)
    raise ValueError(f"unsupported tensor type {ttype}")


def scales_finite(ttype, raw, rows, cols):
    """True when every block scale of a quantized tensor is finite."""
    if ttype == T_F32:
        return True
    bb = 34 if ttype == T_Q8_0 else 18
    b = np.frombuffer(np.asarray(raw, dtype=np.uint8).tobytes(), dtype=np.uint8).reshape(rows, _nblk(cols), bb)
    e = (b[:, :, 1] >> 2) & 0x1F
    return bool(np.all(e != 31))
