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

K-quants (GGUF's public layout too; ggml ids Q4_K = 12, Q6_K = 14): 256-value
super-blocks, a row holds cols/256 of them (cols a multiple of 256).
  Q4_K (144 B): fp16 d, fp16 dmin, 12 bytes of eight 6-bit (scale, min)
    pairs, 128 bytes of 4-bit quants.  Sub-block j (values 32j..32j+31) has
      j < 4:  sc = s[j] & 63,                      m = s[j + 4] & 63
      j >= 4: sc = (s[j + 4] & 15) | (s[j - 4] >> 6) << 4,
              m  = (s[j + 4] >> 4) | (s[j] >> 6) << 4
    and w = d*sc*q - dmin*m.  Quant bytes 32c..32c+31 hold sub-block 2c in
    their low nibbles and sub-block 2c + 1 in their high nibbles.
  Q6_K (210 B): 128 bytes ql (low 4 bits), 64 bytes qh (high 2 bits), sixteen
    int8 scales, fp16 d.  For half h (values 128h..128h+127), l < 32, with
    L = ql[64h..], H = qh[32h..]:
      value 128h + l      : L[l] & 15        | (H[l] & 3) << 4
      value 128h + 32 + l : L[l + 32] & 15   | (H[l] >> 2 & 3) << 4
      value 128h + 64 + l : L[l] >> 4        | (H[l] >> 4 & 3) << 4
      value 128h + 96 + l : L[l + 32] >> 4   | (H[l] >> 6) << 4
    and w = d*scale[i // 16]*(q - 32) for value i of the super-block.
Both products are computed in float64 (exactly) and rounded once to float32.
"""
import numpy as np

T_F32 = 0
T_Q4_0 = 2
T_Q8_0 = 8
T_Q4_K = 12
T_Q6_K = 14
SUPER = {T_Q4_K: 144, T_Q6_K: 210}


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


def _superblocks(raw, rows, cols, ttype):
    if cols % 256:
        raise ValueError(f"K-quant rows need a multiple of 256 values, got {cols}")
    nb = cols // 256
    bb = SUPER[ttype]
    b = np.frombuffer(np.asarray(raw, dtype=np.uint8).tobytes(), dtype=np.uint8)
    if b.size != rows * nb * bb:
        raise ValueError(f"type {ttype}: expected {rows * nb * bb} bytes, got {b.size}")
    return b.reshape(rows * nb, bb)


def _half(lo, hi):
    return _f16_to_f32(lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)).astype(np.float64)


def q4_k_scale_min(s):
    """The eight (scale, min) 6-bit pairs of Q4_K scale bytes s [..., 12]."""
    s = s.astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), np.int64)
    mn = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = s[..., j] & 63
        mn[..., j] = s[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
        mn[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, mn


def dequant_q4_k(raw, rows, cols):
    """Decode Q4_K super-blocks into f32 [rows][cols]."""
    b = _superblocks(raw, rows, cols, T_Q4_K)
    d = _half(b[:, 0], b[:, 1])
    dmin = _half(b[:, 2], b[:, 3])
    sc, mn = q4_k_scale_min(b[:, 4:16])
    qs = b[:, 16:144].reshape(-1, 4, 32)
    q = np.empty((b.shape[0], 8, 32), np.float64)
    q[:, 0::2, :] = qs & 15      # sub-blocks 0, 2, 4, 6: low nibbles
    q[:, 1::2, :] = qs >> 4      # sub-blocks 1, 3, 5, 7: high nibbles
    w = d[:, None, None] * sc[:, :, None] * q - dmin[:, None, None] * mn[:, :, None]
    return w.reshape(rows, cols).astype(np.float32)


def dequant_q6_k(raw, rows, cols):
    """Decode Q6_K super-blocks into f32 [rows][cols]."""
    b = _superblocks(raw, rows, cols, T_Q6_K)
    n = b.shape[0]
    ql = b[:, 0:128].astype(np.int64).reshape(n, 2, 64)
    qh = b[:, 128:192].astype(np.int64).reshape(n, 2, 32)
    scale = b[:, 192:208].view(np.int8).astype(np.float64)
    d = _half(b[:, 208], b[:, 209])
    q = np.empty((n, 2, 4, 32), np.int64)
    q[:, :, 0] = (ql[:, :, :32] & 15) | ((qh & 3) << 4)
    q[:, :, 1] = (ql[:, :, 32:] & 15) | (((qh >> 2) & 3) << 4)
    q[:, :, 2] = (ql[:, :, :32] >> 4) | (((qh >> 4) & 3) << 4)
    q[:, :, 3] = (ql[:, :, 32:] >> 4) | ((qh >> 6) << 4)
    q = q.reshape(n, 256).astype(np.float64) - 32.0
    w = d[:, None] * np.repeat(scale, 16, axis=1) * q
    return w.reshape(rows, cols).astype(np.float32)


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
    if ttype == T_Q4_K:
        return dequant_q4_k(raw, rows, cols)
    if ttype == T_Q6_K:
        return dequant_q6_k(raw, rows, cols)
    raise ValueError(f"unsupported tensor type {ttype}")


def scales_finite(ttype, raw, rows, cols):
    """True when every block scale of a quantized tensor is finite."""
    if ttype == T_F32:
        return True
    if ttype in SUPER:
        b = _superblocks(raw, rows, cols, ttype)
        his = [b[:, 1], b[:, 3]] if ttype == T_Q4_K else [b[:, 209]]
        return all(bool(np.all(((h >> 2) & 0x1F) != 31)) for h in his)
    bb = 34 if ttype == T_Q8_0 else 18
    b = np.frombuffer(np.asarray(raw, dtype=np.uint8).tobytes(), dtype=np.uint8).reshape(rows, _nblk(cols), bb)
    e = (b[:, :, 1] >> 2) & 0x1F
    return bool(np.all(e != 31))
