"""The decoder forward pass over a KV cache, prefill and decode, in float64.

Op order of one block follows the qwen3 architecture file printed in Synsema
"Local inference and architectures", section "The format" (embed; per layer
rms_norm, q/k/v matmuls, per-head norm of q and k, rope, attention, output
matmul, residual add, rms_norm, gate, silu, up, mul, down, residual add; then
the final rms_norm, the last position, and the LM head taken from
output.weight, or token_embd.weight when that is absent), and the Qwen3-0.6B
walkthrough's Steps 2-9 ("How Modern LLMs Actually Generate Text").

Readings where the pages are silent (each also listed in the design notes):
  * the causal rule with a non-empty cache: the query at absolute position p
    sees keys j <= p (the page's triu mask is only right for an empty cache);
  * sliding-window layers see keys p - window < j <= p; layer i is global iff
    i % window_period == window_period - 1; local layers use rope_theta_local;
  * sandwich norms: RMSNorm of each sublayer output (own gain) before its
    residual add;
  * q/k/v biases (qwen2, which the same page says differs from llama only by
    its three bias lines): each added to its projection's output, before the
    per-head norm and RoPE;
  * positions are absolute: a call appends at kv_len and advances it.

Weights are decoded exactly (``oracle.blocks``) and all arithmetic is float64,
except the RoPE angle which the walkthrough computes in float32.
"""
import numpy as np

from . import blocks
from . import ops

F64 = np.float64


class OracleModel:
    """A plain CPU decoder.  ``tensors`` maps GGUF names to objects with
    ``type``, ``rows``, ``cols`` and ``data`` (raw bytes)."""

    def __init__(self, cfg, tensors, max_ctx, n_seqs=1, cache_weights=True):
        self.cfg = dict(cfg)
        self.t = tensors
        self.max_ctx = int(max_ctx)
        self.n_seqs = int(n_seqs)
        self.cache_weights = cache_weights
        self._w = {}
        c = self.cfg
        self.nq, self.nkv, self.hd = c["n_head"], c["n_head_kv"], c["head_dim"]
        self.kv = [[None] * c["n_layer"] for _ in range(self.n_seqs)]
        self.kv_len = [0] * self.n_seqs
        self.inv_freq_global = ops.rope_inv_freq(c["rope_theta"], self.hd)
        self.inv_freq_local = ops.rope_inv_freq(c.get("rope_theta_local", c["rope_theta"]), self.hd)

    # ------------------------------------------------------------ weights
    def mat(self, name):
        """Decoded tensor as float64 [rows][cols] (gains: [cols])."""
        if name in self._w:
            return self._w[name]
        t = self.t[name]
        w = blocks.dequant(t.type, t.data, t.rows, t.cols).astype(F64)
        if t.rows == 1 and not name.endswith("embd.weight") and name != "output.weight":
            w = w.reshape(-1)
        if self.cache_weights:
            self._w[name] = w
        return w

    def lm_head_name(self):
        return "output.weight" if "output.weight" in self.t else "token_embd.weight"

    def embed(self, tokens):
        """Rows of token_embd for the given ids (only those rows are decoded)."""
        t = self.t["token_embd.weight"]
        raw = np.frombuffer(np.asarray(t.data, dtype=np.uint8).tobytes(), dtype=np.uint8)
        row_bytes = raw.size // t.rows
        rows = raw.reshape(t.rows, row_bytes)[np.asarray(tokens, dtype=np.int64)]
        return blocks.dequant(t.type, rows.reshape(-1), len(tokens), t.cols).astype(F64)

    # ------------------------------------------------------------ state
    def reset(self, seq=-1):
        seqs = range(self.n_seqs) if seq < 0 else [seq]
        for s in seqs:
            self.kv_len[s] = 0
            self.kv[s] = [None] * self.cfg["n_layer"]

    def _cache(self, seq, layer):
        if self.kv[seq][layer] is None:
            shape = (self.nkv, self.max_ctx, self.hd)
            self.kv[seq][layer] = (np.zeros(shape, F64), np.zeros(shape, F64))
        return self.kv[seq][layer]

    def kv_write(self, seq, layer, k, v):
        """Install preset post-RoPE K/V [n_kv][n_pos][hd] at positions 0..n_pos-1."""
        K, V = self._cache(seq, layer)
        n = k.shape[1]
        K[:, :n] = k
        V[:, :n] = v

    def set_kv_len(self, seq, n):
        self.kv_len[seq] = int(n)

    def is_global(self, layer):
        c = self.cfg
        if c["window"] <= 0:
            return True
        return layer % c["window_period"] == c["window_period"] - 1

    # ------------------------------------------------------------ forward
    def hidden(self, seq, tokens):
        """Run the blocks over ``tokens`` appended at kv_len; return the final
        residual x [T][H] (before the output norm) and advance kv_len."""
        c = self.cfg
        tokens = np.asarray(tokens, dtype=np.int64)
        T = len(tokens)
        p0 = self.kv_len[seq]
        if p0 + T > self.max_ctx:
            raise ValueError("context overflow")
        pos = np.arange(p0, p0 + T)
        eps = c["rms_eps"]
        nq, nkv, hd = self.nq, self.nkv, self.hd
        act = ops.ACTS[c["act"]]
        x = self.embed(tokens)
        for l in range(c["n_layer"]):
            p = f"blk.{l}."
            h = ops.rmsnorm(x, self.mat(p + "attn_norm.weight"), eps)
            q = h @ self.mat(p + "attn_q.weight").T
            k = h @ self.mat(p + "attn_k.weight").T
            v = h @ self.mat(p + "attn_v.weight").T
            if c.get("qkv_bias"):
                q = q + self.mat(p + "attn_q.bias")
                k = k + self.mat(p + "attn_k.bias")
                v = v + self.mat(p + "attn_v.bias")
            q = q.reshape(T, nq, hd).transpose(1, 0, 2)
            k = k.reshape(T, nkv, hd).transpose(1, 0, 2)
            v = v.reshape(T, nkv, hd).transpose(1, 0, 2)
            if c["qk_norm"]:
                q = ops.rmsnorm(q, self.mat(p + "attn_q_norm.weight"), eps)
                k = ops.rmsnorm(k, self.mat(p + "attn_k_norm.weight"), eps)
            glob = self.is_global(l)
            ang = ops.rope_angles(pos, self.inv_freq_global if glob else self.inv_freq_local)
            q = ops.apply_rope(q, ang)
            k = ops.apply_rope(k, ang)
            K, V = self._cache(seq, l)
            K[:, p0:p0 + T] = k
            V[:, p0:p0 + T] = v
            o = ops.attention(q, K[:, :p0 + T], V[:, :p0 + T], pos, 0 if glob else c["window"])
            a = o.transpose(1, 0, 2).reshape(T, nq * hd)
            y = a @ self.mat(p + "attn_output.weight").T
            if c["sandwich_norm"]:
                y = ops.rmsnorm(y, self.mat(p + "post_attention_norm.weight"), eps)
            x = x + y
            h = ops.rmsnorm(x, self.mat(p + "ffn_norm.weight"), eps)
            m = act(h @ self.mat(p + "ffn_gate.weight").T) * (h @ self.mat(p + "ffn_up.weight").T)
            y = m @ self.mat(p + "ffn_down.weight").T
            if c["sandwich_norm"]:
                y = ops.rmsnorm(y, self.mat(p + "post_ffw_norm.weight"), eps)
            x = x + y
        self.kv_len[seq] = p0 + T
        return x

    def head(self, x):
        """Final RMSNorm and LM head: logits [rows][vocab] (float64)."""
        xn = ops.rmsnorm(x, self.mat("output_norm.weight"), self.cfg["rms_eps"])
        return xn @ self.mat(self.lm_head_name()).T

    def forward(self, seq, tokens, all_logits=False):
        """Append ``tokens`` to sequence ``seq``; logits of the last position
        ([1][V]) or of every position ([T][V])."""
        x = self.hidden(seq, tokens)
        return self.head(x if all_logits else x[-1:])

    def decode(self, tokens):
        """One step for sequences 0..len(tokens)-1, one token each: logits [B][V]."""
        return np.concatenate([self.forward(s, [int(t)]) for s, t in enumerate(tokens)], axis=0)
