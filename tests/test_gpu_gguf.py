"""GPU parity of models loaded from GGUF files (qdec_load_gguf): the library
reads the file with its own reader and compiles the architecture definition
into its fused block; the oracle reads the same file with its own reader and
runs the same definition statement by statement.  Every prefill and decode
logits row within 2e-3 (max |gpu - oracle| / max |oracle|); greedy tokens as
in the other parity tests, decode continuing by teacher forcing."""
import numpy as np
import pytest

import synth
import synth.gguf as sg
from oracle import archdef as ad
from oracle import gguf
from tests.gpu_helpers import SMALL, as_np, check_row, token_agrees

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import decoder_gguf_quantized_amd as qdec  # noqa: E402

REORDERED_QWEN2 = """arch qwen2
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


def cfg_for(key, **kw):
    c = dict(SMALL[key])
    c["ffn"] = (c["ffn"] + 31) // 32 * 32
    c.update(kw)
    return c


# (case, config, definition text or None for the library's built-in)
CASES = {
    "llama_q4": (cfg_for("llama_q4_hd64_g4"), None),
    "qwen3": (cfg_for("qwen3_hd128_g2"), None),
    "qwen2_bias": (cfg_for("qwen2_bias_hd64_g2"), None),
    "qwen2_reordered": (cfg_for("qwen2_bias_hd64_g2"), REORDERED_QWEN2),
    "gemma3_pattern3": (cfg_for("gemma_hd256_g4"),
                        sg.archdef_text("gemma3").replace("window_pattern 6", "window_pattern 3")),
    "gemma3_builtin_7l": (cfg_for("gemma_hd256_g4", n_layer=7, window_period=6, name="gemma_7l"), None),
    "llama_q4_k_m": (cfg_for("q4km_mixed_hd64_g4"), None),
}


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("case", sorted(CASES))
def test_gguf_model_matches_the_interpreted_definition(tmp_path, case):
    cfg, text = CASES[case]
    path = sg.write(str(tmp_path / f"{case}.gguf"), cfg, synth.generate(cfg))
    print(f"case {case}: {path}", flush=True)
    dev()
    T, n = 40, 8
    prompt = synth.prompt(cfg, T)
    V = cfg["vocab"]
    with qdec.Model.from_gguf(path, text, max_seqs=1, max_ctx=64) as m:
        assert m.vocab == V
        pl = torch.empty((T, V), dtype=torch.float32, device=dev())
        tok = torch.empty(1, dtype=torch.int32, device=dev())
        m.prefill(0, prompt, pl, tok, all_logits=True)
        dl = torch.empty((n, V), dtype=torch.float32, device=dev())
        toks = torch.empty((n, 1), dtype=torch.int32, device=dev())
        cur = tok
        for s in range(n):
            m.decode_step(cur, dl[s:s + 1], toks[s])
            cur = toks[s]
        torch.cuda.synchronize()
        g_pl, g_dl = as_np(pl), as_np(dl)
        g_tok = [int(as_np(tok)[0])] + as_np(toks).reshape(-1).tolist()
    src = text if text is not None else sg.archdef_text(sg.arch_of(cfg))
    it = ad.Interpreter(ad.parse(src), gguf.read(path), max_ctx=T + n + 1)
    o_pl = it.forward(0, prompt, all_logits=True)
    o_dl = [it.forward(0, [g_tok[s]])[0] for s in range(n)]
    errs = [check_row(g_pl[i], o_pl[i]) for i in range(T)]
    errs += [check_row(g_dl[s], o_dl[s]) for s in range(n)]
    assert token_agrees(g_tok[0], o_pl[-1])
    for s in range(n):
        assert token_agrees(g_tok[s + 1], o_dl[s])
    print(f"{case}: max rel err {max(errs):.2e}")


def test_refused_definition_leaves_no_handle(tmp_path):
    cfg = cfg_for("llama_q4_hd64_g4")
    path = sg.write(str(tmp_path / "m.gguf"), cfg, synth.generate(cfg))
    dev()
    with pytest.raises(qdec.QdecError, match="layout"):
        qdec.Model.from_gguf(path, sg.archdef_text("llama").replace("silu(g)", "relu(g)"))
