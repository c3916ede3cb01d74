"""Pins for oracle.archdef: the grammar of architecture definitions and the
literal interpreter, checked against the pinned flag-driven OracleModel on
every shipped architecture and against closed forms (CPU only)."""
import numpy as np
import pytest

import synth
import synth.gguf as sg
from oracle import OracleModel
from oracle import archdef as ad
from oracle import gguf


def cfg_for(key, **kw):
    from tests.gpu_helpers import SMALL
    c = dict(SMALL[key])
    c["ffn"] = (c["ffn"] + 31) // 32 * 32
    c.update(kw)
    return c


def gemma_text(pattern):
    return sg.archdef_text("gemma3").replace("window_pattern 6", f"window_pattern {pattern}")


# ---------------------------------------------------------------- grammar
def test_parse_shipped_definitions():
    for arch in ("llama", "qwen2", "qwen3", "gemma3"):
        d = ad.parse(sg.archdef_text(arch), arch)
        assert d.arch == arch and d.kind == "decoder"
        assert [s.op for s in d.sections["prologue"]] == ["embed"]
        assert [s.op for s in d.sections["epilogue"]] == ["rms_norm", "last", "matmul"]
        assert d.sections["epilogue"][2].args == ["x", "output.weight | token_embd.weight"]
    g = ad.parse(sg.archdef_text("gemma3"))
    assert g.params == {"window_pattern": "6", "rope_freq_base_local": "10000"}
    ops = [s.op for s in g.sections["block"]]
    assert ops.count("rms_norm") == 4 and "gelu_tanh" in ops and ops.count("norm_heads") == 2
    q2 = [s for s in ad.parse(sg.archdef_text("qwen2")).sections["block"] if s.op == "add_bias"]
    assert [(s.dst, s.args[1], s.inplace) for s in q2] == [
        ("q", "blk.{i}.attn_q.bias", True), ("k", "blk.{i}.attn_k.bias", True), ("v", "blk.{i}.attn_v.bias", True)]


BAD = [
    ("kind decoder\nblock\n  add(x, x)\n", "no arch"),
    ("arch a\nkind encoder\nblock\n  add(x, x)\n", "kind"),
    ("arch a\nkind decoder\nblock\n  frob(x)\n", "unknown operation"),
    ("arch a\nkind decoder\nblock\n  add(x)\n", "takes 2"),
    ("arch a\nkind decoder\nblock\n  attention(q, k, v)\n", "destination"),
    ("arch a\nkind decoder\nblock\n  x = matmul(h, nodot)\n", "tensor name"),
    ("arch a\nkind decoder\nblock\n  x = matmul(a.b, t.w)\n", "register"),
    ("arch a\nkind decoder\nparam colour red\nblock\n  add(x, x)\n", "unknown param"),
    ("arch a\nkind decoder\nblock\n  add(x, x)\nprologue\n  x = embed(t.w)\n", "out of order"),
    ("arch a\nkind decoder\nprologue\n  x = embed(t.w)\n", "no block"),
    ("arch a\nkind decoder\nblock\n  x = add(x, x\n", "not a statement"),
]


@pytest.mark.parametrize("text,msg", BAD)
def test_parse_refusals(text, msg):
    with pytest.raises(ad.ArchdefError, match=msg):
        ad.parse(text)


def test_file_name_must_be_the_arch():
    with pytest.raises(ad.ArchdefError, match="declares arch llama"):
        ad.parse(sg.archdef_text("llama"), "qwen3")


# ---------------------------------------------------------------- interpreter
def run_both(cfg, text, tmp_path, toks=9, steps=3):
    t = synth.generate(cfg)
    p = sg.write(str(tmp_path / "m.gguf"), cfg, t)
    it = ad.Interpreter(ad.parse(text), gguf.read(p), max_ctx=32)
    om = OracleModel(cfg, t, max_ctx=32)
    pr = synth.prompt(cfg, toks)
    outs = [(it.forward(0, pr, all_logits=True), om.forward(0, pr, all_logits=True))]
    for s in range(steps):
        tok = [int(np.argmax(outs[-1][1][-1]))]
        outs.append((it.decode(tok), om.decode(tok)))
    return outs


@pytest.mark.parametrize("key,text", [
    ("llama_q4_hd64_g4", None), ("qwen3_hd128_g2", None), ("qwen2_bias_hd64_g2", None),
    ("gemma_hd256_g4", gemma_text(3)), ("gqa8_hd128", None)])
def test_interpreter_equals_the_oracle_model(tmp_path, key, text):
    """Each shipped definition, run statement by statement over the GGUF file,
    reproduces the flag-driven OracleModel on the tensors it was written from
    (prefill logits of every position, then greedy decode steps)."""
    cfg = cfg_for(key)
    text = text or sg.archdef_text(sg.arch_of(cfg))
    for a, b in run_both(cfg, text, tmp_path):
        assert np.max(np.abs(a - b)) <= 1e-10 * np.max(np.abs(b))


def test_reordered_definition_computes_the_same(tmp_path):
    """Register names, statement order and in-place / assigned forms do not
    change what a definition computes."""
    cfg = cfg_for("qwen2_bias_hd64_g2")
    text = """arch qwen2
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
  logits = matmul(y, output.weight | token_embd.weight)
  logits = last(logits)
"""
    for a, b in run_both(cfg, text, tmp_path, steps=1):
        assert np.max(np.abs(a - b)) <= 1e-10 * np.max(np.abs(b))


def test_scale_and_head_alternatives(tmp_path):
    """scale(x, c) after the embedding equals a model whose embedding rows are
    c times larger (c = 2, exact in f32); a head naming only token_embd.weight
    ignores output.weight."""
    cfg = cfg_for("llama_q4_hd64_g4", embd_type="f32", wtype="f32")
    t = synth.generate(cfg)
    p = sg.write(str(tmp_path / "m.gguf"), cfg, t)
    g = gguf.read(p)
    base = sg.archdef_text("llama")
    scaled = base.replace("x = embed(token_embd.weight)\n", "x = embed(token_embd.weight)\n  scale(x, 2)\n")
    t2 = dict(t)
    e = t["token_embd.weight"]
    e2 = (np.frombuffer(e.data.tobytes(), np.float32) * np.float32(2.0)).astype(np.float32)
    t2["token_embd.weight"] = synth.SynthTensor(e.name, e.type, e.rows, e.cols, e2.view(np.uint8).copy())
    p2 = sg.write(str(tmp_path / "m2.gguf"), cfg, t2)
    pr = synth.prompt(cfg, 6)
    a = ad.Interpreter(ad.parse(scaled), g, 16).forward(0, pr, all_logits=True)
    # the LM head reads output.weight here, so only the embedding changed
    b = ad.Interpreter(ad.parse(base), gguf.read(p2), 16).forward(0, pr, all_logits=True)
    assert np.max(np.abs(a - b)) <= 1e-10 * np.max(np.abs(b))
    tied_text = base.replace("output.weight | token_embd.weight", "token_embd.weight")
    c = ad.Interpreter(ad.parse(tied_text), g, 16).forward(0, pr)
    om_tied = OracleModel(cfg, {k: v for k, v in t.items() if k != "output.weight"}, 16).forward(0, pr)
    assert np.max(np.abs(c - om_tied)) <= 1e-10 * np.max(np.abs(om_tied))


def test_definition_and_file_must_agree(tmp_path):
    cfg = cfg_for("llama_q4_hd64_g4")
    g = gguf.read(sg.write(str(tmp_path / "m.gguf"), cfg, synth.generate(cfg)))
    with pytest.raises(ad.ArchdefError, match="the file is"):
        ad.Interpreter(ad.parse(sg.archdef_text("qwen3")), g, 8)
    cfg = cfg_for("gemma_hd256_g4")
    g = gguf.read(sg.write(str(tmp_path / "g.gguf"), cfg, synth.generate(cfg)))
    no_pattern = gemma_text(3).replace("param window_pattern 3\n", "")
    with pytest.raises(ad.ArchdefError, match="window_pattern"):
        ad.Interpreter(ad.parse(no_pattern), g, 8)
