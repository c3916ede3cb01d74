"""Model shapes and run recipes of the five seeded synthetic workloads.

Each entry describes a decoder by its shape only; the weights are drawn by
``synth.generate``.  Field meanings:

  n_layer, hidden, n_head, n_head_kv, head_dim, ffn, vocab -- the usual shape
  rms_eps            -- RMSNorm epsilon (1e-6 everywhere, as in the Qwen3
                        walkthrough's RMSNorm step)
  rope_theta         -- RoPE base of full-attention layers
  rope_theta_local   -- RoPE base of sliding-window layers (window > 0 only)
  window, window_period -- sliding window length; layer i is global iff
                        i % window_period == window_period - 1
  qk_norm            -- per-head RMSNorm of Q and K before RoPE (Qwen3)
  qkv_bias           -- the q, k and v projections add a bias (Qwen2); absent = False
  sandwich_norm      -- RMSNorm of each sublayer output before its residual add
  act                -- "silu" (SwiGLU) or "gelu_tanh" (GeGLU)
  wtype              -- block type of every 2-D layer matrix
  embd_type          -- block type of token_embd.weight
  tied               -- LM head reuses token_embd.weight (no output.weight)
  seed               -- generator seed
  prompt_len, decode_steps, batch -- the run recipe
  temperature        -- 0 = greedy
  preset_kv          -- positions of preset K/V per sequence (batched decode)
"""

TINY = dict(
    name="tiny-llama-2L-h256", n_layer=2, hidden=256, n_head=4, n_head_kv=2, head_dim=64,
    ffn=688, vocab=1024, rms_eps=1e-6, rope_theta=1e4, rope_theta_local=1e4,
    window=0, window_period=0, qk_norm=False, sandwich_norm=False, act="silu",
    wtype="q8_0", embd_type="f32", tied=True, seed=1,
    prompt_len=16, decode_steps=16, batch=1, temperature=0.0, preset_kv=0,
)

QWEN3_06B = dict(
    name="qwen3-0.6b-shape", n_layer=28, hidden=1024, n_head=16, n_head_kv=8, head_dim=128,
    ffn=3072, vocab=151936, rms_eps=1e-6, rope_theta=1e6, rope_theta_local=1e6,
    window=0, window_period=0, qk_norm=True, sandwich_norm=False, act="silu",
    wtype="q8_0", embd_type="q8_0", tied=True, seed=2,
    prompt_len=512, decode_steps=256, batch=1, temperature=0.0, preset_kv=0,
)

LLAMA_8B = dict(
    name="llama-8b-shape", n_layer=32, hidden=4096, n_head=32, n_head_kv=8, head_dim=128,
    ffn=14336, vocab=128256, rms_eps=1e-6, rope_theta=5e5, rope_theta_local=5e5,
    window=0, window_period=0, qk_norm=False, sandwich_norm=False, act="silu",
    wtype="q4_0", embd_type="q4_0", tied=False, seed=3,
    prompt_len=1024, decode_steps=128, batch=1, temperature=0.0, preset_kv=0,
)

GEMMA3_1B = dict(
    name="gemma-3-1b-shape", n_layer=26, hidden=1152, n_head=4, n_head_kv=1, head_dim=256,
    ffn=6912, vocab=262144, rms_eps=1e-6, rope_theta=1e6, rope_theta_local=1e4,
    window=512, window_period=6, qk_norm=True, sandwich_norm=True, act="gelu_tanh",
    wtype="q8_0", embd_type="q8_0", tied=True, seed=4,
    prompt_len=2048, decode_steps=128, batch=1, temperature=0.0, preset_kv=0,
)

QWEN3_06B_BATCH16 = dict(
    QWEN3_06B, name="qwen3-0.6b-shape-b16-kv8192", seed=5,
    prompt_len=0, decode_steps=64, batch=16, temperature=1.0, preset_kv=8192,
)

CONFIGS = {
    "c1": TINY,
    "c2": QWEN3_06B,
    "c3": LLAMA_8B,
    "c4": GEMMA3_1B,
    "c5": QWEN3_06B_BATCH16,
}


def get(name):
    """Return a copy of the named configuration ("c1".."c5")."""
    return dict(CONFIGS[name.lower()])


def layer_is_global(cfg, i):
    """True when layer i attends over the whole prefix (no sliding window)."""
    if cfg["window"] <= 0:
        return True
    return i % cfg["window_period"] == cfg["window_period"] - 1
