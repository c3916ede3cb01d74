"""Host-only checks of the library's model-file path (qdec_gguf_config,
qdec_archdef_builtin): the C++ GGUF reader and the architecture-definition
compiler, on files the synthetic-input writer makes and on the hand-laid
fixture.  No GPU work."""
import os
import struct

import pytest

import decoder_gguf_quantized_amd as qdec
import synth
import synth.gguf as sg

HERE = os.path.dirname(os.path.abspath(__file__))
ARCHS = ("llama", "qwen2", "qwen3", "gemma3")
SHAPE_KEYS = ("n_layer", "hidden", "n_head", "n_head_kv", "head_dim", "ffn", "vocab", "window", "window_period",
              "qk_norm", "sandwich_norm", "qkv_bias", "act")


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(qdec.lib_path()):
        from decoder_gguf_quantized_amd import build
        build.build()


def cfg_for(key, **kw):
    from tests.gpu_helpers import SMALL
    c = dict(SMALL[key])
    c["ffn"] = (c["ffn"] + 31) // 32 * 32
    c.update(kw)
    return c


CASES = {"llama": "llama_q4_hd64_g4", "qwen2": "qwen2_bias_hd64_g2", "qwen3": "qwen3_hd128_g2",
         "gemma3": "gemma_hd256_g4"}


@pytest.fixture(scope="module")
def files(tmp_path_factory):
    d = tmp_path_factory.mktemp("gguf")
    out = {}
    for arch, key in CASES.items():
        cfg = cfg_for(key, window_period=6) if arch == "gemma3" else cfg_for(key)
        out[arch] = (cfg, sg.write(str(d / f"{arch}.gguf"), cfg, synth.generate(cfg)))
    return out


def same_shape(got, cfg):
    for k in SHAPE_KEYS:
        assert got[k] == (cfg[k] if k != "qkv_bias" else bool(cfg.get("qkv_bias"))), k
    for k in ("rms_eps", "rope_theta", "rope_theta_local"):
        assert abs(got[k] - cfg[k]) <= 1e-6 * abs(cfg[k]), k


@pytest.mark.parametrize("arch", ARCHS)
def test_builtin_definition_gives_the_written_shape(files, arch):
    cfg, path = files[arch]
    same_shape(qdec.gguf_config(path), cfg)


@pytest.mark.parametrize("arch", ARCHS)
def test_shipped_text_compiles_like_the_builtin(files, arch):
    """The definition files beside the synthetic inputs and the library's
    built-in texts describe the same layouts."""
    cfg, path = files[arch]
    assert qdec.gguf_config(path, sg.archdef_text(arch)) == qdec.gguf_config(path)
    assert qdec.archdef_builtin(arch).startswith(f"arch {arch}\n")


def test_builtins():
    assert qdec.archdef_builtin("mamba") is None
    assert "window_pattern 6" in qdec.archdef_builtin("gemma3")


REORDERED = """arch qwen2
kind decoder
prologue
  x = embed(token_embd.weight)
block
  n = rms_norm(x, blk.{i}.attn_norm.weight)
  vv = matmul(n, blk.{i}.attn_v.weight)
  kk = matmul(n, blk.{i}.attn_k.weight)
  qq = matmul(n, blk.{i}.attn_q.weight)
  add_bias(vv, blk.{i}.attn_v.bias)
  qq = add_bias(qq, blk.{i}.attn_q.bias)
  add_bias(kk, blk.{i}.attn_k.bias)
  rope(kk, head_count_kv)
  rope(qq, head_count)
  att = attention(qq, kk, vv)
  out = matmul(att, blk.{i}.attn_output.weight)
  x = add(out, x)
  n = rms_norm(x, blk.{i}.ffn_norm.weight)
  up = matmul(n, blk.{i}.ffn_up.weight)
  gate = matmul(n, blk.{i}.ffn_gate.weight)
  gate = silu(gate)
  mul(up, gate)
  dn = matmul(up, blk.{i}.ffn_down.weight)
  add(x, dn)
epilogue
  y = copy(x)
  y = rms_norm(y, output_norm.weight)
  y = last(y)
  logits = matmul(y, output.weight | token_embd.weight)
"""


def test_equivalent_definition_is_accepted(files):
    """Register names, statement order and in-place / assigned forms do not
    matter to the compiler; what is computed does."""
    cfg, path = files["qwen2"]
    assert qdec.gguf_config(path, REORDERED) == qdec.gguf_config(path)


def variants(text):
    """Definitions that compute something the kernels do not run."""
    return {
        "relu gate": text.replace("silu(g)", "relu(g)"),
        "exact gelu": text.replace("silu(g)", "gelu(g)"),
        "no rope on k": text.replace("  rope(k, head_count_kv)\n", ""),
        "bias after rope": text.replace("  add_bias(q, blk.{i}.attn_q.bias)\n", "").replace(
            "  rope(q, head_count)\n", "  rope(q, head_count)\n  add_bias(q, blk.{i}.attn_q.bias)\n"),
        "gate and up swapped": text.replace("blk.{i}.ffn_gate.weight", "TMP").replace(
            "blk.{i}.ffn_up.weight", "blk.{i}.ffn_gate.weight").replace("TMP", "blk.{i}.ffn_up.weight"),
        "second residual missing": text.replace("  add(x, d)\n", ""),
        "scaled embedding": text.replace("x = embed(token_embd.weight)\n",
                                         "x = embed(token_embd.weight)\n  scale(x, 2)\n"),
        "no final norm": text.replace("  x = rms_norm(x, output_norm.weight)\n", ""),
        "unknown register": text.replace("a = attention(q, k, v)", "a = attention(q, k, w)"),
        "unknown op": text.replace("silu(g)", "swish(g)"),
    }


@pytest.mark.parametrize("name", list(variants(sg.archdef_text("qwen2"))))
def test_unsupported_definitions_are_refused(files, name):
    _, path = files["qwen2"]
    text = variants(sg.archdef_text("qwen2"))[name]
    with pytest.raises(qdec.QdecError):
        qdec.gguf_config(path, text)


def test_file_and_definition_must_agree(files):
    _, path = files["llama"]
    with pytest.raises(qdec.QdecError, match="architecture is 'llama'"):
        qdec.gguf_config(path, sg.archdef_text("qwen3"))
    _, gpath = files["gemma3"]
    no_pattern = sg.archdef_text("gemma3").replace("param window_pattern 6\n", "")
    with pytest.raises(qdec.QdecError, match="window_pattern"):
        qdec.gguf_config(gpath, no_pattern)
    with pytest.raises(qdec.QdecError, match="lacks"):
        qdec.gguf_config(files["qwen3"][1], sg.archdef_text("qwen3").replace(
            "output.weight | token_embd.weight", "output.weight"))


def golden_bytes():
    txt = open(os.path.join(HERE, "golden", "tiny.gguf.hex")).read()
    return bytes(int(x, 16) for ln in txt.splitlines() for x in ln.split("#")[0].split())


def test_hand_laid_file_parses_up_to_the_model_shape(tmp_path):
    """The library reads the whole container of the hand-laid file (metadata of
    three kinds, two tensors, alignment padding) and stops at the first shape
    key the llama definition needs."""
    p = tmp_path / "tiny.gguf"
    p.write_bytes(golden_bytes())
    with pytest.raises(qdec.QdecError, match="'llama.block_count' is missing"):
        qdec.gguf_config(str(p))


@pytest.mark.parametrize("patch,msg", [
    (lambda b: b"GGUG" + b[4:], "magic"),
    (lambda b: b[:4] + struct.pack("<I", 1) + b[8:], "version"),
    (lambda b: b[:206] + struct.pack("<Q", 33) + b[214:], "multiple"),
    (lambda b: b[:206] + struct.pack("<Q", 64) + b[214:], "end of the file"),
    (lambda b: b[:186] + struct.pack("<Q", 31) + b[194:], "blocks"),
    (lambda b: b.replace(b"llama.rope.freq_base", b"general.architecture"), "twice"),
    (lambda b: b[:150], "ends inside"),
    (lambda b: b[:20], "too short|ends inside"),
])
def test_corrupt_files_are_refused(tmp_path, patch, msg):
    p = tmp_path / "bad.gguf"
    p.write_bytes(patch(golden_bytes()))
    with pytest.raises(qdec.QdecError, match=msg):
        qdec.gguf_config(str(p))


def test_k_quant_rows_must_hold_whole_super_blocks(tmp_path):
    """A Q4_K tensor whose rows are not a multiple of 256 values cannot be laid
    out; the writer refuses it, and a patched file is refused by the reader."""
    from tests.gpu_helpers import SMALL
    cfg = dict(SMALL["q4km_mixed_hd64_g4"])
    t = synth.generate(cfg)
    p = sg.write(str(tmp_path / "k.gguf"), cfg, t)
    b = open(p, "rb").read()
    # token_embd.weight's ne[0] = 512 -> 500: the reader's row-length check
    key = b"token_embd.weight"
    at = b.index(key) + len(key) + 4
    assert struct.unpack("<Q", b[at:at + 8])[0] == 512
    bad = tmp_path / "bad.gguf"
    bad.write_bytes(b[:at] + struct.pack("<Q", 500) + b[at + 8:])
    with pytest.raises(qdec.QdecError, match="256"):
        qdec.gguf_config(str(bad))
    assert qdec.gguf_config(p)["hidden"] == 512


def test_missing_file_and_null_arguments(tmp_path):
    with pytest.raises(qdec.QdecError, match="cannot open"):
        qdec.gguf_config(str(tmp_path / "none.gguf"))
    L = qdec.lib()
    assert L.qdec_gguf_config(None, None, None) == 1
    assert L.qdec_load_gguf(None, None, 1, 16, None, None) == 1


def test_every_name_in_a_definition_must_resolve(files):
    """Statements whose results are never used are still checked: their
    tensors must be in the file (in every layer, for the block), their numbers
    numbers or metadata keys, and {i} appears only in the block."""
    _, path = files["qwen3"]
    text = sg.archdef_text("qwen3")
    dead_missing = text.replace("block\n", "block\n  z = rms_norm(x, blk.{i}.no_such.weight)\n")
    with pytest.raises(qdec.QdecError, match="'blk.0.no_such.weight' is not in the file"):
        qdec.gguf_config(path, dead_missing)
    dead_short = text.replace("block\n", "block\n  z = rms_norm(x, output_norm.weight)\n")
    assert qdec.gguf_config(path, dead_short) == qdec.gguf_config(path)
    epi_layer = text.replace("epilogue\n", "epilogue\n  z = rms_norm(x, blk.{i}.attn_norm.weight)\n")
    with pytest.raises(qdec.QdecError, match=r"\{i\} names a layer only inside the block"):
        qdec.gguf_config(path, epi_layer)
    dead_number = text.replace("block\n", "block\n  z = scale(x, no_such_key)\n")
    with pytest.raises(qdec.QdecError, match="neither a number nor a metadata key"):
        qdec.gguf_config(path, dead_number)
    dead_key = text.replace("block\n", "block\n  z = scale(x, block_count)\n  w = scale(x, 0.5)\n")
    assert qdec.gguf_config(path, dead_key) == qdec.gguf_config(path)


def test_block_tensors_resolve_in_every_layer(tmp_path):
    """A tensor that only layer 0 has fails at layer 1 when the block names it."""
    cfg = cfg_for("qwen3_hd128_g2")
    assert cfg["n_layer"] >= 2
    t = synth.generate(cfg)
    t["blk.0.extra.weight"] = t["blk.0.attn_norm.weight"]
    order = [s[0] for s in sg.tensor_specs(cfg)] + ["blk.0.extra.weight"]
    path = sg.write(str(tmp_path / "x.gguf"), cfg, t, order=order)
    text = sg.archdef_text("qwen3")
    assert qdec.gguf_config(path, text) == qdec.gguf_config(path)
    with pytest.raises(qdec.QdecError, match="'blk.1.extra.weight' is not in the file"):
        qdec.gguf_config(path, text.replace("block\n", "block\n  z = rms_norm(x, blk.{i}.extra.weight)\n"))
