"""Pins for oracle.gguf (the oracle's GGUF reader): a file laid out by hand from
the container definition, round trips of files the synthetic-input writer
makes, and the refusals (CPU only)."""
import os
import struct

import numpy as np
import pytest

import synth
import synth.gguf as sg
from oracle import blocks
from oracle import gguf

HERE = os.path.dirname(os.path.abspath(__file__))


def golden_bytes():
    """tests/golden/tiny.gguf.hex: a 290-byte file laid out field by field."""
    txt = open(os.path.join(HERE, "golden", "tiny.gguf.hex")).read()
    return bytes(int(x, 16) for ln in txt.splitlines() for x in ln.split("#")[0].split())


def test_hand_laid_file():
    b = golden_bytes()
    assert len(b) == 290
    g = gguf.read_bytes(b)
    assert g.version == 3 and g.alignment == 32 and g.data_start == 224
    assert g.metadata == {"general.architecture": "llama", "llama.rope.freq_base": 10000.0, "t.arr": [-2, 3]}
    a, w = g.tensors["a"], g.tensors["b.w"]
    assert (a.type, a.ne, a.rows, a.cols, a.offset) == (0, (4,), 1, 4, 0)
    assert np.frombuffer(a.data.tobytes(), "<f4").tolist() == [1.0, -2.0, 0.5, 3.0]
    assert (w.type, w.ne, w.rows, w.cols, w.offset) == (8, (32, 1), 1, 32, 32)
    assert blocks.dequant(8, w.data, 1, 32).reshape(-1).tolist() == [0.25 * (j - 16) for j in range(32)]


def cfg_for(key):
    from tests.gpu_helpers import SMALL
    c = dict(SMALL[key])
    c["ffn"] = (c["ffn"] + 31) // 32 * 32
    return c


@pytest.mark.parametrize("key,alignment,shuffle", [("llama_q4_hd64_g4", 32, False), ("qwen2_bias_hd64_g2", 64, True),
                                                   ("gemma_hd256_g4", 256, False)])
def test_round_trip_of_written_files(tmp_path, key, alignment, shuffle):
    cfg = cfg_for(key)
    t = synth.generate(cfg)
    order = None
    if shuffle:
        order = [s[0] for s in synth.tensor_specs(cfg)]
        np.random.default_rng(0).shuffle(order)
    p = sg.write(str(tmp_path / "m.gguf"), cfg, t, alignment=alignment, order=order)
    g = gguf.read(p)
    assert g.alignment == alignment and g.data_start % alignment == 0
    assert set(g.tensors) == set(t)
    for n, st in t.items():
        gt = g.tensors[n]
        assert (gt.type, gt.rows, gt.cols) == (st.type, st.rows, st.cols), n
        assert gt.offset % alignment == 0
        assert np.array_equal(gt.data, st.data), n
    arch = sg.arch_of(cfg)
    md = g.metadata
    assert md["general.architecture"] == arch
    assert md[f"{arch}.block_count"] == cfg["n_layer"]
    assert md[f"{arch}.attention.head_count_kv"] == cfg["n_head_kv"]
    assert md[f"{arch}.attention.layer_norm_rms_epsilon"] == np.float32(cfg["rms_eps"])
    assert md["tokenizer.ggml.tokens"][:3] == ["<t0>", "<t1>", "<t2>"]
    assert len(md["tokenizer.ggml.scores"]) == cfg["vocab"]
    assert md["general.tags"] == [["synthetic", "seeded"], [1, 2, 3]]
    assert md["general.quantized"] is True


def test_refusals():
    b = golden_bytes()
    with pytest.raises(gguf.GGUFError, match="magic"):
        gguf.read_bytes(b"GGUG" + b[4:])
    with pytest.raises(gguf.GGUFError, match="version"):
        gguf.read_bytes(b[:4] + struct.pack("<I", 1) + b[8:])
    for cut in (3, 20, 100, 150, 200, 289):
        with pytest.raises(gguf.GGUFError):
            gguf.read_bytes(b[:cut])
    # b.w's offset 32 -> 33: not a multiple of the alignment
    off = 214 - 8
    assert struct.unpack("<Q", b[off:off + 8])[0] == 32
    with pytest.raises(gguf.GGUFError, match="multiple"):
        gguf.read_bytes(b[:off] + struct.pack("<Q", 33) + b[off + 8:])
    # b.w's row of 32 values -> 31: not whole blocks
    ne0 = 171 + 8 + 3 + 4
    with pytest.raises(gguf.GGUFError, match="blocks"):
        gguf.read_bytes(b[:ne0] + struct.pack("<Q", 31) + b[ne0 + 8:])
    # offset 64 runs past the end
    with pytest.raises(gguf.GGUFError, match="end of the file"):
        gguf.read_bytes(b[:off] + struct.pack("<Q", 64) + b[off + 8:])
    # the second metadata key renamed to the first: a duplicate
    dup = b.replace(b"llama.rope.freq_base", b"general.architecture")
    with pytest.raises(gguf.GGUFError, match="twice"):
        gguf.read_bytes(dup)
