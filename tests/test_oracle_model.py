"""Pins for oracle.model: closed forms on hand-built models and invariants on
seeded ones (CPU only)."""
import math

import numpy as np
import pytest

import synth
from oracle import OracleModel, ops

TINY = dict(name="pin", n_layer=2, hidden=16, n_head=4, n_head_kv=2, head_dim=4, ffn=12, vocab=10,
            rms_eps=1e-6, rope_theta=1e4, rope_theta_local=1e4, window=0, window_period=0,
            qk_norm=False, sandwich_norm=False, act="silu", wtype="f32", embd_type="f32", tied=True,
            seed=7, prompt_len=6, decode_steps=3, batch=1, temperature=0.0, preset_kv=0)


def f32_model(cfg, fill):
    """Tensors of ``cfg`` as f32 records; fill(name, rows, cols) -> array."""
    out = {}
    for name, _t, rows, cols, _k in synth.tensor_specs(cfg):
        a = np.asarray(fill(name, rows, cols), dtype=np.float32).reshape(rows, cols)
        out[name] = synth.SynthTensor(name, synth.T_F32, rows, cols, a.view(np.uint8).reshape(-1).copy())
    return out


def rand_embed_zero_rest(seed):
    r = np.random.default_rng(seed)

    def fill(name, rows, cols):
        if name == "token_embd.weight":
            return r.standard_normal((rows, cols))
        if rows == 1:
            return 1 + 0.1 * r.standard_normal(cols)
        return np.zeros((rows, cols))
    return fill


def test_zero_layers_pass_residual_through():
    m_t = f32_model(TINY, rand_embed_zero_rest(1))
    m = OracleModel(TINY, m_t, max_ctx=8)
    toks = [3, 0, 9, 3]
    logits = m.forward(0, toks, all_logits=True)
    E = np.frombuffer(m_t["token_embd.weight"].data.tobytes(), np.float32).reshape(10, 16).astype(np.float64)
    g = np.frombuffer(m_t["output_norm.weight"].data.tobytes(), np.float32).astype(np.float64)
    for i, t in enumerate(toks):
        e = E[t]
        xn = e / math.sqrt(np.mean(e * e) + 1e-6) * g
        assert np.allclose(logits[i], E @ xn, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("rv,head", [(5, 0), (5, 2), (5, 3), (2, 1), (2, 3)])
def test_one_hot_v_and_o_with_uniform_attention(rv, head):
    """Q = K = 0 makes attention uniform over the prefix.  attn_v one-hot at
    (rv, cv) and attn_output one-hot at (ro, co) give, per position t,
    x_t[ro] += wo * mean_{j<=t}(wv * h_j[cv]) iff column co reads a query head of
    the KV head that owns rv (GQA by repeat).  Pins the orientation of attn_v
    (8 x 16) and of the square attn_output (16 x 16), and the head mapping."""
    cfg = dict(TINY, n_layer=1)
    hd, group = 4, 2
    g_kv = rv // hd
    co = head * hd + rv % hd
    reads = head // group == g_kv
    cv, ro, wv, wo = 11, 6, 0.75, -1.25
    base = rand_embed_zero_rest(2)

    def fill(name, rows, cols):
        if name.endswith("attn_v.weight"):
            a = np.zeros((rows, cols)); a[rv, cv] = wv; return a
        if name.endswith("attn_output.weight"):
            a = np.zeros((rows, cols)); a[ro, co] = wo; return a
        return base(name, rows, cols)
    t = f32_model(cfg, fill)
    m = OracleModel(cfg, t, max_ctx=8)
    toks = [1, 4, 4, 7, 2]
    x = m.hidden(0, toks)
    E = np.frombuffer(t["token_embd.weight"].data.tobytes(), np.float32).reshape(10, 16).astype(np.float64)
    ga = np.frombuffer(t["blk.0.attn_norm.weight"].data.tobytes(), np.float32).astype(np.float64)
    h = np.array([E[k] / math.sqrt(np.mean(E[k] ** 2) + 1e-6) * ga for k in toks])
    for i in range(len(toks)):
        want = E[toks[i]].copy()
        if reads:
            want[ro] += wo * np.mean(wv * h[:i + 1, cv])
        assert np.allclose(x[i], want, rtol=1e-13, atol=1e-14)


def test_window_one_makes_every_position_independent():
    """Window 1 on every layer: each position attends only to itself, so the
    logits of a token do not depend on its position or neighbours, except through
    RoPE, which cancels for a query against its own key."""
    cfg = dict(TINY, window=1, window_period=100, qk_norm=True)
    t = synth.generate(dict(cfg, wtype="q8_0"), threads=1)
    m = OracleModel(cfg, t, max_ctx=16)
    a = m.forward(0, [5, 2, 7, 2, 9, 5], all_logits=True)
    assert np.allclose(a[1], a[3], rtol=1e-12)
    assert np.allclose(a[0], a[5], rtol=1e-12)
    m.reset()
    b = m.forward(0, [2], all_logits=True)
    assert np.allclose(a[1], b[0], rtol=1e-12)


VARIANTS = {
    "llama": dict(TINY, wtype="q8_0"),
    "qwen3": dict(TINY, wtype="q8_0", qk_norm=True, rope_theta=1e6, rope_theta_local=1e6),
    "gemma3": dict(TINY, wtype="q8_0", qk_norm=True, sandwich_norm=True, act="gelu_tanh",
                   window=3, window_period=2, rope_theta=1e6, rope_theta_local=1e4, n_head_kv=1),
    "q4": dict(TINY, wtype="q4_0", embd_type="q4_0", tied=False, ffn=40),
}


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_kv_cached_decode_equals_full_recompute(variant):
    cfg = VARIANTS[variant]
    t = synth.generate(cfg, threads=1)
    toks = list(synth.prompt(cfg, 9))
    full = OracleModel(cfg, t, max_ctx=16).forward(0, toks, all_logits=True)
    m = OracleModel(cfg, t, max_ctx=16)
    rows = [m.forward(0, toks[:4], all_logits=True)]
    for tok in toks[4:]:
        rows.append(m.forward(0, [tok]))
    inc = np.concatenate(rows, axis=0)
    assert np.allclose(inc, full, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_causality(variant):
    cfg = VARIANTS[variant]
    t = synth.generate(cfg, threads=1)
    toks = list(synth.prompt(cfg, 8))
    a = OracleModel(cfg, t, max_ctx=16).forward(0, toks, all_logits=True)
    toks2 = toks[:5] + [(x + 1) % cfg["vocab"] for x in toks[5:]]
    b = OracleModel(cfg, t, max_ctx=16).forward(0, toks2, all_logits=True)
    assert np.array_equal(a[:5], b[:5])
    assert not np.allclose(a[5:], b[5:])


def test_split_prefill_equals_single_prefill():
    cfg = VARIANTS["qwen3"]
    t = synth.generate(cfg, threads=1)
    toks = list(synth.prompt(cfg, 10))
    one = OracleModel(cfg, t, max_ctx=16).forward(0, toks)
    m = OracleModel(cfg, t, max_ctx=16)
    m.forward(0, toks[:6])
    two = m.forward(0, toks[6:])
    assert np.allclose(one, two, rtol=1e-11, atol=1e-13)


def test_sequences_are_independent_and_reset_reproduces():
    cfg = VARIANTS["llama"]
    t = synth.generate(cfg, threads=1)
    m = OracleModel(cfg, t, max_ctx=16, n_seqs=2)
    a = m.forward(0, [1, 2, 3])
    m.forward(1, [4, 4, 4, 4])
    b = m.forward(0, [5])
    m.reset(0)
    assert np.array_equal(m.forward(0, [1, 2, 3]), a)
    assert np.array_equal(m.forward(0, [5]), b)


def test_untied_head_uses_output_weight():
    cfg = VARIANTS["q4"]
    t = synth.generate(cfg, threads=1)
    m = OracleModel(cfg, t, max_ctx=8)
    assert m.lm_head_name() == "output.weight"
    tied = OracleModel(VARIANTS["llama"], synth.generate(VARIANTS["llama"], threads=1), max_ctx=8)
    assert tied.lm_head_name() == "token_embd.weight"


def test_quantized_embedding_rows_match_full_decode():
    cfg = VARIANTS["q4"]
    t = synth.generate(cfg, threads=1)
    m = OracleModel(cfg, t, max_ctx=8)
    from oracle import blocks
    te = t["token_embd.weight"]
    full = blocks.dequant(te.type, te.data, te.rows, te.cols)
    assert np.array_equal(m.embed([3, 0, 3]), full[[3, 0, 3]].astype(np.float64))


def test_rmsnorm_and_rope_order_in_block():
    """Per-head norm happens before RoPE: with an all-equal gain the order does
    not matter (RoPE keeps the head's norm), with a non-uniform gain it does."""
    x = np.random.default_rng(3).standard_normal((1, 1, 8))
    ang = ops.rope_angles([3], ops.rope_inv_freq(1e4, 8))
    w1 = np.full(8, 1.3)
    a = ops.apply_rope(ops.rmsnorm(x, w1, 1e-6), ang)
    b = ops.rmsnorm(ops.apply_rope(x, ang), w1, 1e-6)
    assert np.allclose(a, b, rtol=1e-12)
    w2 = np.linspace(0.5, 2.0, 8)
    a = ops.apply_rope(ops.rmsnorm(x, w2, 1e-6), ang)
    b = ops.rmsnorm(ops.apply_rope(x, ang), w2, 1e-6)
    assert not np.allclose(a, b)


# ---------------------------------------------------------------- q/k/v biases (qwen2)
BIAS = dict(TINY, n_layer=1, qkv_bias=True)


def bias_fill(seed, zero=(), bias_override=None):
    """Random f32 tensors; names ending in an entry of ``zero`` are all zeros;
    ``bias_override`` maps a bias name suffix to a fixed vector."""
    r = np.random.default_rng(seed)
    bias_override = bias_override or {}

    def fill(name, rows, cols):
        for suffix, vec in bias_override.items():
            if name.endswith(suffix):
                return np.asarray(vec, dtype=np.float64).reshape(rows, cols)
        if any(name.endswith(z) for z in zero):
            return np.zeros((rows, cols))
        if name.endswith(".bias"):
            return r.standard_normal((rows, cols))
        if rows == 1:
            return 1 + 0.1 * r.standard_normal((rows, cols))
        return r.standard_normal((rows, cols))
    return fill


def f32_of(t):
    return np.frombuffer(t.data.tobytes(), np.float32).astype(np.float64).reshape(t.rows, t.cols)


def test_v_bias_with_zero_v_weight_is_the_attention_output():
    """attn_v = 0 makes every value row equal b_v; the softmax weights of any
    query sum to one, so each query head's attention output is b_v of its KV
    head whatever q, k and their biases are.  With ffn_down = 0 as well the
    residual after the layer is embed + W_o (b_v repeated over each query
    group), at every position."""
    t = f32_model(BIAS, bias_fill(3, zero=("attn_v.weight", "ffn_down.weight")))
    m = OracleModel(BIAS, t, max_ctx=8)
    toks = [4, 1, 7, 7, 2]
    x = m.hidden(0, toks)
    E = f32_of(t["token_embd.weight"])
    bv = f32_of(t["blk.0.attn_v.bias"]).reshape(BIAS["n_head_kv"], BIAS["head_dim"])
    group = BIAS["n_head"] // BIAS["n_head_kv"]
    a = np.repeat(bv, group, axis=0).reshape(-1)
    want = E[toks] + a @ f32_of(t["blk.0.attn_output.weight"]).T
    assert np.allclose(x, want, rtol=1e-12, atol=1e-12)


def test_zero_biases_equal_the_model_without_biases():
    cfg_b = dict(TINY, qkv_bias=True)
    zero = {s: np.zeros(n) for s, n in (("attn_q.bias", 16), ("attn_k.bias", 8), ("attn_v.bias", 8))}
    tb = f32_model(cfg_b, bias_fill(5, bias_override=zero))
    tn = f32_model(TINY, bias_fill(5))
    toks = [1, 2, 3, 9, 0]
    lb = OracleModel(cfg_b, tb, max_ctx=8).forward(0, toks, all_logits=True)
    ln = OracleModel(TINY, tn, max_ctx=8).forward(0, toks, all_logits=True)
    assert np.array_equal(lb, ln)


def test_q_bias_is_irrelevant_when_keys_are_zero_and_k_bias_is_not():
    """attn_k = 0 and b_k = 0 make every key zero, so every score is zero and
    the q bias cannot move the output; a non-zero b_k makes the scores depend
    on the q bias again."""
    toks = [5, 5, 8, 0, 3, 1]
    zk = {"attn_k.bias": np.zeros(8)}

    def run(bq, bk):
        over = {"attn_q.bias": bq}
        if bk is not None:
            over["attn_k.bias"] = bk
        t = f32_model(BIAS, bias_fill(9, zero=("attn_k.weight",), bias_override=over))
        return OracleModel(BIAS, t, max_ctx=8).forward(0, toks, all_logits=True)

    r = np.random.default_rng(1)
    bq1, bq2, bk = 3 * r.standard_normal(16), 3 * r.standard_normal(16), 3 * r.standard_normal(8)
    assert np.array_equal(run(bq1, zk["attn_k.bias"]), run(bq2, zk["attn_k.bias"]))
    d = np.max(np.abs(run(bq1, bk) - run(bq2, bk)))
    assert d > 1e-3


def _post_norm_gains(name, cols):
    """Distinct gains for the two sublayer post-norms, so that taking the other
    sublayer's gain changes the result at every index."""
    if name.endswith("post_attention_norm.weight"):
        return np.linspace(0.5, 2.0, cols)
    if name.endswith("post_ffw_norm.weight"):
        return np.linspace(2.25, 0.75, cols)
    return None


def _post_normed_one_hot(y, gain, H, eps):
    """RMSNorm of a vector whose only non-zero entry is y: mean square y^2 / H,
    so the entry becomes gain * y / sqrt(y^2 / H + eps) (about sign(y) sqrt(H)
    gain when y^2 >> H eps) and every other entry stays 0."""
    return gain * y / math.sqrt(y * y / H + eps)


@pytest.mark.parametrize("rv,head", [(5, 2), (2, 1)])
def test_sandwich_attention_post_norm_closed_form(rv, head):
    """Gemma-3 block reading (sandwich norms): the attention sublayer's output
    W_o a is RMS-normalised with its own gain post_attention_norm and only then
    added to the residual.  With Q = K = 0 (uniform attention), attn_v one-hot at
    (rv, cv) and attn_output one-hot at (ro, co), the sublayer output is a
    one-hot vector y e_ro with y = wo * mean_{j<=i}(wv h_j[cv]); its RMSNorm is
    the closed form above, so x_i = e_{t_i} + that at ro.  The zero FFN adds
    RMSNorm(0) = 0.  A norm after the residual add, the FFN's gain, a norm of
    the attention output before W_o, or no norm all give other values."""
    cfg = dict(TINY, n_layer=1, sandwich_norm=True)
    H, hd = 16, 4
    co = head * hd + rv % hd
    cv, ro, wv, wo = 11, 6, 0.75, -1.25
    base = rand_embed_zero_rest(3)

    def fill(name, rows, cols):
        if name.endswith("attn_v.weight"):
            a = np.zeros((rows, cols)); a[rv, cv] = wv; return a
        if name.endswith("attn_output.weight"):
            a = np.zeros((rows, cols)); a[ro, co] = wo; return a
        g = _post_norm_gains(name, cols)
        return g if g is not None else base(name, rows, cols)
    t = f32_model(cfg, fill)
    m = OracleModel(cfg, t, max_ctx=8)
    toks = [1, 4, 4, 7, 2]
    x = m.hidden(0, toks)
    E = np.frombuffer(t["token_embd.weight"].data.tobytes(), np.float32).reshape(10, 16).astype(np.float64)
    ga = np.frombuffer(t["blk.0.attn_norm.weight"].data.tobytes(), np.float32).astype(np.float64)
    gpa = np.linspace(0.5, 2.0, H).astype(np.float32).astype(np.float64)
    h = np.array([E[k] / math.sqrt(np.mean(E[k] ** 2) + 1e-6) * ga for k in toks])
    for i in range(len(toks)):
        want = E[toks[i]].copy()
        y = wo * np.mean(wv * h[:i + 1, cv])
        want[ro] += _post_normed_one_hot(y, gpa[ro], H, 1e-6)
        assert np.allclose(x[i], want, rtol=1e-12, atol=1e-13)
        # the one-hot post-norm is about sign(y) sqrt(H) gain: far from y itself
        assert abs(x[i][ro] - E[toks[i]][ro]) > 3.0 * abs(y)


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_sandwich_ffn_post_norm_closed_form(act):
    """The FFN sublayer's output is RMS-normalised with post_ffw_norm before its
    residual add.  Zero attention (attn_v = 0: the post-attention norm of a zero
    vector is 0), ffn_gate and ffn_up one-hot in row kf (columns c1, c2) and
    ffn_down one-hot at (ro, kf): per position m[kf] = act(wg h[c1]) (wu h[c2])
    with h = RMSNorm(e_t, ffn_norm), the FFN output is wd m[kf] e_ro, and
    x = e_t + (its one-hot RMSNorm) at ro."""
    cfg = dict(TINY, n_layer=1, sandwich_norm=True, act=act)
    H = 16
    kf, c1, c2, ro = 7, 3, 12, 9
    wg, wu, wd = 1.5, -0.75, 0.625  # exact in f32
    base = rand_embed_zero_rest(4)

    def fill(name, rows, cols):
        a = np.zeros((rows, cols))
        if name.endswith("ffn_gate.weight"):
            a[kf, c1] = wg; return a
        if name.endswith("ffn_up.weight"):
            a[kf, c2] = wu; return a
        if name.endswith("ffn_down.weight"):
            a[ro, kf] = wd; return a
        g = _post_norm_gains(name, cols)
        return g if g is not None else base(name, rows, cols)
    t = f32_model(cfg, fill)
    m = OracleModel(cfg, t, max_ctx=8)
    toks = [0, 5, 5, 8]
    x = m.hidden(0, toks)
    E = np.frombuffer(t["token_embd.weight"].data.tobytes(), np.float32).reshape(10, 16).astype(np.float64)
    gf = np.frombuffer(t["blk.0.ffn_norm.weight"].data.tobytes(), np.float32).astype(np.float64)
    gpf = np.linspace(2.25, 0.75, H).astype(np.float32).astype(np.float64)

    def f(g):
        if act == "silu":
            return g / (1.0 + math.exp(-g))
        return 0.5 * g * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (g + 0.044715 * g ** 3)))
    for i, tok in enumerate(toks):
        e = E[tok]
        h = e / math.sqrt(np.mean(e * e) + 1e-6) * gf
        y = wd * f(wg * h[c1]) * (wu * h[c2])
        want = e.copy()
        want[ro] += _post_normed_one_hot(y, gpf[ro], H, 1e-6)
        assert np.allclose(x[i], want, rtol=1e-12, atol=1e-13)
