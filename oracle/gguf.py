"""GGUF container reader -- TEST INFRASTRUCTURE (part of the oracle).

Reads the file a GGUF model ships in, as the public GGUF specification lays
it out (versions 2 and 3, little-endian): the magic "GGUF", the version, the
tensor and metadata counts (u64), the metadata (key string, u32 value type,
value), the tensor infos (name, u32 n_dims, u64 ne[n_dims] with ne[0] the
contiguous dimension, u32 ggml type, u64 offset), then the tensor data from
the next multiple of the alignment (general.alignment, else 32), each
tensor's offset counted from there.  A string is a u64 byte length and its
bytes; an array is a u32 element type, a u64 count and the elements.

Plain and slow on purpose: every field is read with ``struct`` in file order.
It shares nothing with the GPU library's reader.  The tensor types the
decoder uses are F32 (0), Q4_0 (2), Q8_0 (8), Q4_K (12) and Q6_K (14); other
types are read as opaque records with their byte size unknown and refused
when used.
"""
import struct
from dataclasses import dataclass, field

import numpy as np

_SCALARS = {0: ("<B", 1), 1: ("<b", 1), 2: ("<H", 2), 3: ("<h", 2), 4: ("<I", 4), 5: ("<i", 4),
            6: ("<f", 4), 7: ("<?", 1), 10: ("<Q", 8), 11: ("<q", 8), 12: ("<d", 8)}
T_STRING, T_ARRAY = 8, 9
BLOCK_BYTES = {8: 34, 2: 18}
SUPER_BYTES = {12: 144, 14: 210}  # Q4_K, Q6_K: 256-value super-blocks


class GGUFError(ValueError):
    pass


@dataclass
class GTensor:
    name: str
    type: int
    rows: int          # product of ne[1:] (1 for a vector)
    cols: int          # ne[0]
    ne: tuple
    offset: int        # from the start of the data section
    data: np.ndarray = None  # uint8 bytes of the tensor


@dataclass
class GGUF:
    version: int
    metadata: dict
    tensors: dict = field(default_factory=dict)
    alignment: int = 32
    data_start: int = 0


class _Cursor:
    def __init__(self, buf):
        self.b = buf
        self.p = 0

    def take(self, n):
        if n < 0 or self.p + n > len(self.b):
            raise GGUFError(f"file ends inside a field at byte {self.p} (needs {n} more)")
        out = self.b[self.p:self.p + n]
        self.p += n
        return out

    def scalar(self, fmt, size):
        return struct.unpack(fmt, self.take(size))[0]

    def u32(self):
        return self.scalar("<I", 4)

    def u64(self):
        return self.scalar("<Q", 8)

    def string(self):
        n = self.u64()
        try:
            return bytes(self.take(n)).decode("utf-8")
        except UnicodeDecodeError as e:
            raise GGUFError(f"string at byte {self.p - n} is not UTF-8") from e

    def value(self, vtype, depth=0):
        if vtype in _SCALARS:
            return self.scalar(*_SCALARS[vtype])
        if vtype == T_STRING:
            return self.string()
        if vtype == T_ARRAY:
            if depth > 4:
                raise GGUFError("arrays nested too deeply")
            etype = self.u32()
            n = self.u64()
            return [self.value(etype, depth + 1) for _ in range(n)]
        raise GGUFError(f"unknown metadata value type {vtype}")


def tensor_nbytes(ttype, ne):
    """Bytes of a tensor of ggml type ``ttype`` and shape ``ne`` (None if the
    type is not one the decoder reads)."""
    n = 1
    for d in ne:
        n *= d
    if ttype == 0:
        return 4 * n
    if ttype in BLOCK_BYTES:
        if ne[0] % 32:
            raise GGUFError(f"row length {ne[0]} is not a whole number of 32-value blocks")
        return n // 32 * BLOCK_BYTES[ttype]
    if ttype in SUPER_BYTES:
        if ne[0] % 256:
            raise GGUFError(f"row length {ne[0]} is not a whole number of 256-value super-blocks")
        return n // 256 * SUPER_BYTES[ttype]
    return None


def read_bytes(buf):
    """Parse a whole GGUF file held in memory (bytes or a uint8 array)."""
    buf = memoryview(bytes(buf)) if not isinstance(buf, (bytes, memoryview)) else memoryview(buf)
    c = _Cursor(buf)
    if bytes(c.take(4)) != b"GGUF":
        raise GGUFError("not a GGUF file (magic)")
    version = c.u32()
    if version not in (2, 3):
        raise GGUFError(f"GGUF version {version} unsupported (2, 3)")
    n_tensors = c.u64()
    n_kv = c.u64()
    md = {}
    for _ in range(n_kv):
        key = c.string()
        if key in md:
            raise GGUFError(f"metadata key {key!r} appears twice")
        md[key] = c.value(c.u32())
    align = md.get("general.alignment", 32)
    if not isinstance(align, int) or align <= 0 or align & (align - 1):
        raise GGUFError(f"general.alignment {align!r} is not a power of two")
    infos = []
    for _ in range(n_tensors):
        name = c.string()
        nd = c.u32()
        if not 1 <= nd <= 4:
            raise GGUFError(f"tensor {name!r}: {nd} dimensions")
        ne = tuple(c.u64() for _ in range(nd))
        ttype = c.u32()
        off = c.u64()
        infos.append((name, ne, ttype, off))
    start = c.p + (-c.p) % align
    g = GGUF(version, md, {}, align, start)
    for name, ne, ttype, off in infos:
        if name in g.tensors:
            raise GGUFError(f"tensor {name!r} appears twice")
        if off % align:
            raise GGUFError(f"tensor {name!r}: offset {off} is not a multiple of {align}")
        nb = tensor_nbytes(ttype, ne)
        data = None
        if nb is not None:
            if start + off + nb > len(buf):
                raise GGUFError(f"tensor {name!r}: data runs past the end of the file")
            data = np.frombuffer(buf[start + off:start + off + nb], dtype=np.uint8)
        rows = 1
        for d in ne[1:]:
            rows *= d
        g.tensors[name] = GTensor(name, ttype, rows, ne[0], ne, off, data)
    return g


def read(path):
    with open(path, "rb") as f:
        return read_bytes(f.read())
