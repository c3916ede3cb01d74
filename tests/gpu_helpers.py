"""Shared pieces of the GPU parity tests: small model shapes that exercise every
kernel variant, the tolerance rule, and oracle/GPU runners."""
import numpy as np

import synth

TOL = 2e-3  # max |gpu - oracle| / max |oracle| per logits row

BASE = dict(rms_eps=1e-6, rope_theta=1e4, rope_theta_local=1e4, window=0, window_period=0, qk_norm=False,
            sandwich_norm=False, qkv_bias=False, act="silu", wtype="q8_0", embd_type="q8_0", tied=True, prompt_len=0,
            decode_steps=0, batch=1, temperature=0.0, preset_kv=0)

# Small models, one per kernel variant: head_dim 64/128/256, query heads per KV
# head 1/2/4/8, Q8_0/Q4_0/F32, tied/untied head, QK-norm, sliding window,
# sandwich norms, gelu_tanh, FFN widths that are not multiples of 32 or 64,
# q/k/v biases, K-quants (mixed per matrix).
SMALL = {
    "qwen3_hd128_g2": dict(BASE, name="qwen3_hd128_g2", n_layer=2, hidden=256, n_head=4, n_head_kv=2, head_dim=128,
                           ffn=512, vocab=5000, qk_norm=True, rope_theta=1e6, rope_theta_local=1e6, seed=11),
    "llama_q4_hd64_g4": dict(BASE, name="llama_q4_hd64_g4", n_layer=2, hidden=512, n_head=8, n_head_kv=2, head_dim=64,
                             ffn=1400, vocab=3000, wtype="q4_0", embd_type="q4_0", tied=False, rope_theta=5e5,
                             rope_theta_local=5e5, seed=12),
    "gemma_hd256_g4": dict(BASE, name="gemma_hd256_g4", n_layer=3, hidden=256, n_head=4, n_head_kv=1, head_dim=256,
                           ffn=640, vocab=2048, window=8, window_period=3, qk_norm=True, sandwich_norm=True,
                           act="gelu_tanh", rope_theta=1e6, rope_theta_local=1e4, seed=13),
    "mha_hd128_g1_f32": dict(BASE, name="mha_hd128_g1_f32", n_layer=1, hidden=256, n_head=2, n_head_kv=2, head_dim=128,
                             ffn=336, vocab=1100, wtype="f32", embd_type="f32", seed=14),
    "gqa8_hd128": dict(BASE, name="gqa8_hd128", n_layer=1, hidden=1024, n_head=8, n_head_kv=1, head_dim=128,
                       ffn=96, vocab=4200, qk_norm=True, seed=15),
    "qwen2_bias_hd64_g2": dict(BASE, name="qwen2_bias_hd64_g2", n_layer=2, hidden=384, n_head=6, n_head_kv=3,
                               head_dim=64, ffn=1024, vocab=3000, qkv_bias=True, embd_type="f32", tied=False,
                               rope_theta=1e6, rope_theta_local=1e6, seed=16),
    # a Q4_K_M-like mix: Q4_K matrices, Q6_K for attn_v, ffn_down and the
    # head (so q, k and v have different types and run as three launches)
    "q4km_mixed_hd64_g4": dict(BASE, name="q4km_mixed_hd64_g4", n_layer=2, hidden=512, n_head=8, n_head_kv=2,
                               head_dim=64, ffn=1024, vocab=3000, wtype="q4_k", embd_type="q4_k", tied=False,
                               types={"attn_v": "q6_k", "ffn_down": "q6_k", "output": "q6_k"}, rope_theta=5e5,
                               rope_theta_local=5e5, seed=17),
    "q6k_tied_hd128": dict(BASE, name="q6k_tied_hd128", n_layer=2, hidden=256, n_head=2, n_head_kv=1,
                           head_dim=128, ffn=512, vocab=2048, wtype="q6_k", embd_type="q6_k", qk_norm=True,
                           rope_theta=1e6, rope_theta_local=1e6, seed=18),
}


def rel_err(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return float(np.max(np.abs(g - o)) / np.max(np.abs(o)))


def check_row(g, o, tol=TOL):
    e = rel_err(g, o)
    assert e <= tol, f"max rel err {e:.3e} > {tol}"
    return e


def token_agrees(gpu_token, o_row, tol=TOL):
    """The GPU's greedy token must equal the oracle's argmax whenever the
    oracle's top-2 margin exceeds twice the tolerance (each side may move by
    tol * max|o|); otherwise either token is a valid answer."""
    o = np.asarray(o_row, dtype=np.float64)
    top2 = np.partition(o, -2)[-2:]
    margin = top2[1] - top2[0]
    tau = tol * np.max(np.abs(o))
    if margin > 2 * tau:
        return int(gpu_token) == int(np.argmax(o))
    return True


def as_np(t):
    return t.detach().cpu().numpy()
