"""Seeded synthetic inputs: model tensors in GGUF block layout, prompts, preset KV.

This module produces inputs only.  It holds none of the forward pass: it draws
normal weights, encodes them into Q8_0 / Q4_0 blocks (the encoder is how a GGUF
file is made offline; the decoder path only ever decodes), and draws token ids.
Both the CPU oracle and the GPU library are fed from here and from nowhere else.

Recipe (per tensor): numpy ``Generator(PCG64(SeedSequence([seed, tag_lo, tag_hi,
chunk])))`` where tag is the first 8 bytes of sha256(tensor name) and chunk
indexes fixed row ranges of about 4M values, so large tensors are drawn in
parallel with a result independent of the thread count.
  * 2-D matrices: N(0, 0.02), then block-encoded in the config's type
  * 1-D gains: 1 + N(0, 0.02), float32
  * 1-D q/k/v biases (qkv_bias): N(0, 0.5), float32
  * prompts: uniform ids in [0, vocab)
  * preset K/V (batched long-context workload): N(0, 1) float32

Block layouts (GGUF's public layout; 32 values per block, blocks run along the
input dimension of each output row, a row padded with zeros to whole blocks):
  Q8_0: little-endian fp16 scale d, then 32 int8 q            -> 34 bytes
  Q4_0: little-endian fp16 scale d, then 16 bytes; byte j holds element j in
        its low nibble and element j+16 in its high nibble, value = d*(n-8)
                                                              -> 18 bytes
  Q4_K, Q6_K: 256-value super-blocks (144 and 210 bytes), rows a multiple of
        256 values; the layouts are written out in the encoders below.
A config may give some matrices another type than ``wtype`` with a ``types``
map from the short tensor name (``attn_v``, ``ffn_down``, ``output``, ...) to a
type name, as mixed files (Q4_K_M) do.
"""
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from . import configs
from .configs import CONFIGS, get, layer_is_global  # noqa: F401

# ggml type ids (the numbering a GGUF file uses)
T_F32 = 0
T_Q4_0 = 2
T_Q8_0 = 8
T_Q4_K = 12
T_Q6_K = 14
TYPE_IDS = {"f32": T_F32, "q4_0": T_Q4_0, "q8_0": T_Q8_0, "q4_k": T_Q4_K, "q6_k": T_Q6_K}
BLOCK = 32
BLOCK_BYTES = {T_Q8_0: 34, T_Q4_0: 18}
SUPER_BYTES = {T_Q4_K: 144, T_Q6_K: 210}

Q8_DTYPE = np.dtype([("d", "<f2"), ("qs", "i1", (32,))])
Q4_DTYPE = np.dtype([("d", "<f2"), ("qs", "u1", (16,))])
assert Q8_DTYPE.itemsize == 34 and Q4_DTYPE.itemsize == 18


@dataclass
class SynthTensor:
    name: str
    type: int          # ggml type id
    rows: int          # output dimension (1 for gains)
    cols: int          # logical input dimension
    data: np.ndarray   # raw bytes, uint8, GGUF block layout

    @property
    def nbytes(self):
        return int(self.data.nbytes)

    def sha256(self):
        return hashlib.sha256(self.data.tobytes()).hexdigest()


def n_blocks(cols):
    return (cols + BLOCK - 1) // BLOCK


def tensor_nbytes(ttype, rows, cols):
    if ttype == T_F32:
        return rows * cols * 4
    if ttype in SUPER_BYTES:
        return rows * (cols // 256) * SUPER_BYTES[ttype]
    return rows * n_blocks(cols) * BLOCK_BYTES[ttype]


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _tag(name):
    h = hashlib.sha256(name.encode()).digest()[:8]
    v = int.from_bytes(h, "little")
    return [v & 0xFFFFFFFF, v >> 32]


def _rng(seed, name, chunk):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed] + _tag(name) + [chunk])))


# ---------------------------------------------------------------- encoders
def encode_q8_0(x):
    """f32 [rows][cols] -> Q8_0 blocks [rows][nblk] (structured, 34 B each).

    Per block: amax = max|x|, d = fp16(amax/127), q = clamp(rint(x/d), -127, 127),
    with x/d taken in f32 against the fp16-rounded d; an all-zero block stores
    d = 0, q = 0.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    nb = n_blocks(cols)
    if nb * BLOCK != cols:
        x = np.concatenate([x, np.zeros((rows, nb * BLOCK - cols), np.float32)], axis=1)
    xb = x.reshape(rows, nb, BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    d16 = (amax / np.float32(127.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, np.float32(1.0), d32)
    q = np.rint(xb / safe[..., None])
    np.clip(q, -127, 127, out=q)
    q[d32 == 0] = 0
    out = np.empty((rows, nb), dtype=Q8_DTYPE)
    out["d"] = d16
    out["qs"] = q.astype(np.int8)
    return out


def encode_q4_0(x):
    """f32 [rows][cols] -> Q4_0 blocks [rows][nblk] (structured, 18 B each).

    Per block: amax = max|x|, d = fp16(amax/8), n = clamp(rint(x/d), -8, 7) + 8;
    byte j = n[j] | n[j+16] << 4.  An all-zero block stores d = 0, n = 8.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    nb = n_blocks(cols)
    if nb * BLOCK != cols:
        x = np.concatenate([x, np.zeros((rows, nb * BLOCK - cols), np.float32)], axis=1)
    xb = x.reshape(rows, nb, BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    d16 = (amax / np.float32(8.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, np.float32(1.0), d32)
    n = np.rint(xb / safe[..., None])
    np.clip(n, -8, 7, out=n)
    n[d32 == 0] = 0
    n = (n + 8).astype(np.uint8)
    out = np.empty((rows, nb), dtype=Q4_DTYPE)
    out["d"] = d16
    out["qs"] = n[..., :16] | (n[..., 16:] << 4)
    return out


def _f16(v):
    return np.asarray(v, dtype=np.float32).astype(np.float16)


def encode_q4_k(x):
    """f32 [rows][cols] (cols % 256 == 0) -> Q4_K bytes [rows * cols/256][144].

    Per 32-value sub-block j: lo = min(x, 0), span = max(x) - lo; scale_j =
    span/15, min_j = -lo.  Per super-block d = fp16(max scale_j / 63), dmin =
    fp16(max min_j / 63); sc_j = rint(scale_j / d), m_j = rint(min_j / dmin),
    both clamped to [0, 63]; q = clamp(rint((x + dmin m_j) / (d sc_j)), 0, 15).
    Layout: fp16 d, fp16 dmin, 12 scale bytes (j < 4: byte j = sc_j | (sc_{j+4}
    >> 4) << 6, byte j+4 = m_j | (m_{j+4} >> 4) << 6; byte j+8 = (sc_{j+4} & 15)
    | (m_{j+4} & 15) << 4), then quant byte 32c + l = q[2c][l] | q[2c+1][l] << 4.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % 256 == 0
    xb = x.reshape(-1, 8, 32).astype(np.float64)
    lo = np.minimum(xb.min(axis=2), 0.0)
    scale = (xb.max(axis=2) - lo) / 15.0
    mins = -lo
    d = _f16(scale.max(axis=1) / 63.0).astype(np.float64)
    dmin = _f16(mins.max(axis=1) / 63.0).astype(np.float64)
    sc = np.clip(np.rint(scale / np.where(d == 0, 1, d)[:, None]), 0, 63).astype(np.int64)
    m = np.clip(np.rint(mins / np.where(dmin == 0, 1, dmin)[:, None]), 0, 63).astype(np.int64)
    step = d[:, None] * sc
    q = np.rint((xb + (dmin[:, None] * m)[:, :, None]) / np.where(step == 0, 1, step)[:, :, None])
    q = np.clip(np.where(step[:, :, None] == 0, 0, q), 0, 15).astype(np.uint8)
    out = np.zeros((xb.shape[0], 144), np.uint8)
    out[:, 0:2] = _f16(d).view(np.uint8).reshape(-1, 2)
    out[:, 2:4] = _f16(dmin).view(np.uint8).reshape(-1, 2)
    for j in range(4):
        out[:, 4 + j] = sc[:, j] | ((sc[:, j + 4] >> 4) << 6)
        out[:, 8 + j] = m[:, j] | ((m[:, j + 4] >> 4) << 6)
        out[:, 12 + j] = (sc[:, j + 4] & 15) | ((m[:, j + 4] & 15) << 4)
    for c in range(4):
        out[:, 16 + 32 * c:48 + 32 * c] = q[:, 2 * c] | (q[:, 2 * c + 1] << 4)
    return out.reshape(-1)


def encode_q6_k(x):
    """f32 [rows][cols] (cols % 256 == 0) -> Q6_K bytes [rows * cols/256][210].

    Per 16-value group g: scale_g = max|x| / 31; per super-block d =
    fp16(max scale_g / 127); s_g = clamp(rint(scale_g / d), 0, 127) (int8);
    q = clamp(rint(x / (d s_g)), -32, 31) + 32 (6 bits).  Layout: 128 bytes of
    low nibbles, 64 bytes of 2-bit high parts, 16 int8 scales, fp16 d; within
    half h (values 128h..128h+127) and l < 32, values 128h + l and
    128h + 64 + l share low byte 64h + l (low / high nibble), values
    128h + 32 + l and 128h + 96 + l share low byte 64h + 32 + l, and the high
    parts of those four sit in bits 0-1, 2-3, 4-5, 6-7 of byte 128 + 32h + l.
    """
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % 256 == 0
    xb = x.reshape(-1, 16, 16).astype(np.float64)
    scale = np.abs(xb).max(axis=2) / 31.0
    d = _f16(scale.max(axis=1) / 127.0).astype(np.float64)
    sg = np.clip(np.rint(scale / np.where(d == 0, 1, d)[:, None]), 0, 127).astype(np.int64)
    step = d[:, None] * sg
    q = np.rint(xb / np.where(step == 0, 1, step)[:, :, None])
    q = (np.clip(np.where(step[:, :, None] == 0, 0, q), -32, 31) + 32).astype(np.int64).reshape(-1, 2, 4, 32)
    out = np.zeros((xb.shape[0], 210), np.uint8)
    for h in range(2):
        out[:, 64 * h:64 * h + 32] = (q[:, h, 0] & 15) | ((q[:, h, 2] & 15) << 4)
        out[:, 64 * h + 32:64 * h + 64] = (q[:, h, 1] & 15) | ((q[:, h, 3] & 15) << 4)
        out[:, 128 + 32 * h:160 + 32 * h] = ((q[:, h, 0] >> 4) | ((q[:, h, 1] >> 4) << 2) |
                                             ((q[:, h, 2] >> 4) << 4) | ((q[:, h, 3] >> 4) << 6))
    out[:, 192:208] = sg.astype(np.int8).view(np.uint8)
    out[:, 208:210] = _f16(d).view(np.uint8).reshape(-1, 2)
    return out.reshape(-1)


def encode(ttype, x):
    """Encode an f32 matrix into raw GGUF bytes (uint8, flat)."""
    x = np.asarray(x, dtype=np.float32)
    if ttype == T_F32:
        return np.ascontiguousarray(x).view(np.uint8).reshape(-1).copy()
    if ttype == T_Q4_K:
        return encode_q4_k(x)
    if ttype == T_Q6_K:
        return encode_q6_k(x)
    blocks = encode_q8_0(x) if ttype == T_Q8_0 else encode_q4_0(x)
    return blocks.view(np.uint8).reshape(-1)


# ---------------------------------------------------------------- tensors
def tensor_specs(cfg):
    """List of (name, type id, rows, cols, kind) for a config, kind in {matrix, gain, bias}."""
    H, hd = cfg["hidden"], cfg["head_dim"]
    qd, kd, F, V = cfg["n_head"] * hd, cfg["n_head_kv"] * hd, cfg["ffn"], cfg["vocab"]
    over = cfg.get("types", {})

    def wt_of(short):
        return TYPE_IDS[over.get(short, cfg["wtype"])]
    specs = [("token_embd.weight", TYPE_IDS[cfg["embd_type"]], V, H, "matrix")]
    for i in range(cfg["n_layer"]):
        p = f"blk.{i}."
        specs += [
            (p + "attn_norm.weight", T_F32, 1, H, "gain"),
            (p + "attn_q.weight", wt_of("attn_q"), qd, H, "matrix"),
            (p + "attn_k.weight", wt_of("attn_k"), kd, H, "matrix"),
            (p + "attn_v.weight", wt_of("attn_v"), kd, H, "matrix"),
        ]
        if cfg.get("qkv_bias"):
            specs += [(p + "attn_q.bias", T_F32, 1, qd, "bias"),
                      (p + "attn_k.bias", T_F32, 1, kd, "bias"),
                      (p + "attn_v.bias", T_F32, 1, kd, "bias")]
        if cfg["qk_norm"]:
            specs += [(p + "attn_q_norm.weight", T_F32, 1, hd, "gain"),
                      (p + "attn_k_norm.weight", T_F32, 1, hd, "gain")]
        specs += [(p + "attn_output.weight", wt_of("attn_output"), H, qd, "matrix")]
        if cfg["sandwich_norm"]:
            specs += [(p + "post_attention_norm.weight", T_F32, 1, H, "gain")]
        specs += [
            (p + "ffn_norm.weight", T_F32, 1, H, "gain"),
            (p + "ffn_gate.weight", wt_of("ffn_gate"), F, H, "matrix"),
            (p + "ffn_up.weight", wt_of("ffn_up"), F, H, "matrix"),
            (p + "ffn_down.weight", wt_of("ffn_down"), H, F, "matrix"),
        ]
        if cfg["sandwich_norm"]:
            specs += [(p + "post_ffw_norm.weight", T_F32, 1, H, "gain")]
    specs += [("output_norm.weight", T_F32, 1, H, "gain")]
    if not cfg["tied"]:
        specs += [("output.weight", wt_of("output"), V, H, "matrix")]
    return specs


def _chunk_rows(cols):
    return max(1, (1 << 22) // max(1, cols))


def _gen_tensor(seed, name, ttype, rows, cols, kind, pool):
    if kind == "gain":
        x = 1.0 + 0.02 * _rng(seed, name, 0).standard_normal(cols, dtype=np.float32)
        return SynthTensor(name, T_F32, 1, cols, x.astype(np.float32).view(np.uint8).copy())
    if kind == "bias":
        x = 0.5 * _rng(seed, name, 0).standard_normal(cols, dtype=np.float32)
        return SynthTensor(name, T_F32, 1, cols, x.astype(np.float32).view(np.uint8).copy())
    cr = _chunk_rows(cols)
    starts = list(range(0, rows, cr))
    row_bytes = tensor_nbytes(ttype, 1, cols)
    out = np.empty(rows * row_bytes, dtype=np.uint8)

    def work(ci):
        r0 = starts[ci]
        r1 = min(rows, r0 + cr)
        x = _rng(seed, name, ci).standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= np.float32(0.02)
        out[r0 * row_bytes:r1 * row_bytes] = encode(ttype, x)

    if pool is None or len(starts) == 1:
        for ci in range(len(starts)):
            work(ci)
    else:
        list(pool.map(work, range(len(starts))))
    return SynthTensor(name, ttype, rows, cols, out)


def generate(cfg, threads=None):
    """Draw every tensor of a config.  Returns {name: SynthTensor}."""
    seed = cfg["seed"]
    specs = tensor_specs(cfg)
    nt = threads or _threads()
    with ThreadPoolExecutor(nt) as pool:
        tensors = {}
        for name, ttype, rows, cols, kind in specs:
            tensors[name] = _gen_tensor(seed, name, ttype, rows, cols, kind, pool)
    return tensors


def prompt(cfg, length=None, tag="prompt"):
    """Prompt token ids, int32, uniform in [0, vocab)."""
    n = cfg["prompt_len"] if length is None else length
    return _rng(cfg["seed"], tag, 0).integers(0, cfg["vocab"], size=n).astype(np.int32)


def first_tokens(cfg):
    """First decode input per sequence of the batched preset-KV workload."""
    return _rng(cfg["seed"], "first", 0).integers(0, cfg["vocab"], size=cfg["batch"]).astype(np.int32)


def preset_kv(cfg, seq, layer, n_pos=None):
    """Preset post-RoPE K and V for one (sequence, layer): two f32 [n_kv][n_pos][head_dim]."""
    n = cfg["preset_kv"] if n_pos is None else n_pos
    shape = (cfg["n_head_kv"], n, cfg["head_dim"])
    r = _rng(cfg["seed"], f"kv.{seq}.{layer}", 0)
    k = r.standard_normal(shape, dtype=np.float32)
    v = r.standard_normal(shape, dtype=np.float32)
    return k, v


def preset_kv_all(cfg, seqs=None, threads=None):
    """Yield (seq, layer, k, v) for every preset cache block, drawn in a thread
    pool a few blocks ahead of the consumer (bounded memory)."""
    seqs = range(cfg["batch"]) if seqs is None else seqs
    jobs = [(s, l) for s in seqs for l in range(cfg["n_layer"])]
    nt = threads or _threads()
    with ThreadPoolExecutor(nt) as pool:
        futs = {}
        ahead = 2 * nt
        for i, (s, l) in enumerate(jobs):
            for j in range(i, min(len(jobs), i + ahead)):
                if j not in futs:
                    futs[j] = pool.submit(preset_kv, cfg, *jobs[j])
            k, v = futs.pop(i).result()
            yield s, l, k, v


def manifest(tensors):
    """{name: sha256} of every tensor's bytes, for reports."""
    return {n: t.sha256() for n, t in tensors.items()}


def weight_bytes(cfg):
    """Bytes of every block-encoded matrix (algorithmic weight traffic of one decode step)."""
    return sum(tensor_nbytes(t, r, c) for _, t, r, c, k in tensor_specs(cfg) if k == "matrix")
