"""Write seeded synthetic models as GGUF files, with architecture definitions.

An input generator only: it lays tensors that ``synth.generate`` drew into the
GGUF container and adds the metadata a loader reads the shape from.  It holds
none of the forward pass.

Container (the public GGUF specification, version 3; every integer and float
little-endian):
  u32 magic "GGUF" | u32 version | u64 tensor count | u64 metadata count
  metadata: string key, u32 value type, value
  tensor infos: string name, u32 n_dims, u64 ne[n_dims] (ne[0] = the
                innermost, contiguous dimension), u32 ggml type, u64 offset
  zero padding up to a multiple of the alignment (general.alignment, else 32)
  tensor data; each tensor's offset, counted from the start of the data, is a
  multiple of the alignment
  string = u64 byte length + UTF-8 bytes (no terminator)
  array  = u32 element type + u64 count + the elements

Metadata written (llama.cpp's key names, "<arch>." prefixed where the
architecture owns the key): block_count, context_length, embedding_length,
feed_forward_length, attention.head_count, attention.head_count_kv,
attention.key_length, attention.value_length,
attention.layer_norm_rms_epsilon, rope.freq_base, and
attention.sliding_window when the model has a window; plus general.* and a
tokenizer vocabulary (strings, scores, token types) so that readers meet
arrays of every kind.

Architecture definitions (``archdefs/*.archdef``) are the text format of
Synsema's "Local inference and architectures" page, section "The format".
"""
import os
import struct

import numpy as np

from . import T_F32, T_Q4_0, T_Q4_K, T_Q6_K, T_Q8_0, tensor_specs

MAGIC = b"GGUF"
# metadata value types
U8, I8, U16, I16, U32, I32, F32, BOOL, STR, ARR, U64, I64, F64 = range(13)
_SCALAR = {U8: "<B", I8: "<b", U16: "<H", I16: "<h", U32: "<I", I32: "<i", F32: "<f", BOOL: "<?",
           U64: "<Q", I64: "<q", F64: "<d"}

ARCHDEF_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "archdefs")


def archdef_text(arch):
    """Text of the architecture definition shipped with the synthetic inputs."""
    with open(os.path.join(ARCHDEF_DIR, arch + ".archdef")) as f:
        return f.read()


def arch_of(cfg):
    """The architecture whose definition describes a synthetic config."""
    if cfg.get("qkv_bias"):
        return "qwen2"
    if cfg["sandwich_norm"]:
        return "gemma3"
    return "qwen3" if cfg["qk_norm"] else "llama"


def _string(s):
    b = s.encode("utf-8")
    return struct.pack("<Q", len(b)) + b


def _value(vtype, v):
    if vtype == STR:
        return _string(v)
    if vtype == ARR:
        etype, items = v
        out = [struct.pack("<IQ", etype, len(items))]
        if etype in _SCALAR and etype != BOOL:
            out.append(np.asarray(items, dtype=np.dtype(_SCALAR[etype])).tobytes())
        else:
            out.extend(_value(etype, it) for it in items)
        return b"".join(out)
    return struct.pack(_SCALAR[vtype], v)


def metadata(cfg, arch, alignment=32, vocab_strings=True):
    """Ordered list of (key, type, value) for a synthetic config."""
    a = arch
    md = [("general.architecture", STR, arch),
          ("general.name", STR, cfg["name"]),
          ("general.file_type", U32, 7),
          ("general.quantized", BOOL, True)]
    if alignment != 32:
        md.append(("general.alignment", U32, alignment))
    md += [(a + ".block_count", U32, cfg["n_layer"]),
           (a + ".context_length", U32, 32768),
           (a + ".embedding_length", U32, cfg["hidden"]),
           (a + ".feed_forward_length", U32, cfg["ffn"]),
           (a + ".attention.head_count", U32, cfg["n_head"]),
           (a + ".attention.head_count_kv", U32, cfg["n_head_kv"]),
           (a + ".attention.key_length", U32, cfg["head_dim"]),
           (a + ".attention.value_length", U32, cfg["head_dim"]),
           (a + ".attention.layer_norm_rms_epsilon", F32, cfg["rms_eps"]),
           (a + ".rope.freq_base", F32, cfg["rope_theta"])]
    if cfg["window"] > 0:
        md.append((a + ".attention.sliding_window", U32, cfg["window"]))
    V = cfg["vocab"]
    md += [("tokenizer.ggml.model", STR, "gpt2"),
           ("tokenizer.ggml.scores", ARR, (F32, [float(-i) for i in range(V)])),
           ("tokenizer.ggml.token_type", ARR, (I32, [1] * V)),
           ("tokenizer.ggml.bos_token_id", U32, 1),
           ("general.seed", I64, int(cfg["seed"])),
           ("general.ratio", F64, 0.5),
           ("general.tags", ARR, (ARR, [(STR, ["synthetic", "seeded"]), (U16, [1, 2, 3])]))]
    if vocab_strings:
        md.append(("tokenizer.ggml.tokens", ARR, (STR, [f"<t{i}>" for i in range(V)])))
    return md


def write(path, cfg, tensors, arch=None, alignment=32, order=None, vocab_strings=True):
    """Write ``tensors`` ({name: SynthTensor}) of ``cfg`` as a GGUF file.

    Block-quantized matrices need a row length that is a multiple of 32 (a
    GGUF row holds whole blocks).  ``order`` permutes the tensor list (a
    reader must not depend on it).  Returns the path."""
    arch = arch or arch_of(cfg)
    names = [s[0] for s in tensor_specs(cfg)] if order is None else list(order)
    infos, blobs, off = [], [], 0
    for n in names:
        t = tensors[n]
        if t.type in (T_Q8_0, T_Q4_0) and t.cols % 32:
            raise ValueError(f"{n}: {t.cols} columns is not a whole number of blocks")
        if t.type in (T_Q4_K, T_Q6_K) and t.cols % 256:
            raise ValueError(f"{n}: {t.cols} columns is not a whole number of super-blocks")
        if t.type not in (T_F32, T_Q8_0, T_Q4_0, T_Q4_K, T_Q6_K):
            raise ValueError(f"{n}: type {t.type}")
        ne = [t.cols] if t.rows == 1 and not n.endswith("embd.weight") and n != "output.weight" else [t.cols, t.rows]
        pad = (-off) % alignment
        if pad:
            blobs.append(b"\0" * pad)
            off += pad
        infos.append(_string(n) + struct.pack("<I", len(ne)) + struct.pack(f"<{len(ne)}Q", *ne)
                     + struct.pack("<IQ", t.type, off))
        raw = np.asarray(t.data, dtype=np.uint8).tobytes()
        blobs.append(raw)
        off += len(raw)
    md = metadata(cfg, arch, alignment, vocab_strings)
    head = [MAGIC, struct.pack("<IQQ", 3, len(names), len(md))]
    head += [_string(k) + struct.pack("<I", vt) + _value(vt, v) for k, vt, v in md]
    head += infos
    head = b"".join(head)
    head += b"\0" * ((-len(head)) % alignment)
    with open(path, "wb") as f:
        f.write(head)
        for b in blobs:
            f.write(b)
    return path
