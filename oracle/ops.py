"""Per-step operations of the decoder forward pass, as plain float64 numpy.

Every function follows the plain definition.  Sources (page title, section):
  * RMSNorm: "How Modern LLMs Actually Generate Text" (Qwen3-0.6B walkthrough),
    Step 3 -- x * rsqrt(mean(x*x) + eps) * w, no mean subtraction, no bias.
  * RoPE: same page, Step 4 -- half-split rotation, freqs = 1/theta^(i/half)
    for i < half, angles = position * freq in float32.
  * Attention: same page, Step 5 -- q.k * head_dim^-1/2, causal mask, softmax,
    weighted sum of V, GQA by repeating each KV head over its query heads.
  * SwiGLU: same page, Step 6 -- silu(gate) * up, silu(g) = g * sigmoid(g).
  * gelu_tanh: Synsema "Local inference and architectures", section
    "The operations" names the tanh approximation of GELU (gelu_pytorch_tanh);
    the formula used is the textbook one.
"""
import math

import numpy as np

F64 = np.float64


def rmsnorm(x, w, eps):
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis (float64)."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=F64)


def rope_inv_freq(theta, head_dim):
    """inv_freq[i] = 1 / theta^(i/half) for i < half, evaluated in float64 by the
    C library's pow and rounded once to float32 (the walkthrough keeps freqs in
    float32)."""
    half = head_dim // 2
    vals = [1.0 / math.pow(theta, i / half) for i in range(half)]
    return np.array(vals, dtype=np.float32)


def rope_angles(positions, inv_freq):
    """angle[p][i] = float32(p) * inv_freq[i], a float32 product as in Step 4."""
    p = np.asarray(positions, dtype=np.float32)
    return (p[:, None] * inv_freq[None, :]).astype(np.float32)


def apply_rope(x, angles):
    """Rotate pairs (d, d + half) of x [..., T, head_dim] by angles [T, half].

    [x1, x2] -> [x1 cos - x2 sin, x1 sin + x2 cos] with cos/sin of the float32
    angle evaluated in float64.
    """
    x = np.asarray(x, dtype=F64)
    half = x.shape[-1] // 2
    a = angles.astype(F64)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def softmax(s, axis=-1):
    """exp(s - max) / sum over the axis; -inf entries get weight 0."""
    s = np.asarray(s, dtype=F64)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def allowed_keys(q_pos, n_keys, window):
    """Boolean [T][n_keys]: key j is visible to the query at absolute position p
    iff j <= p, and additionally j > p - window when window > 0."""
    p = np.asarray(q_pos)[:, None]
    j = np.arange(n_keys)[None, :]
    ok = j <= p
    if window > 0:
        ok &= j > p - window
    return ok


def attention(q, k, v, q_pos, window=0):
    """Grouped-query attention.

    q [n_head][T][hd], k and v [n_kv][n_keys][hd] (all keys held so far, post
    RoPE), q_pos [T] absolute positions of the queries.  Query head h reads KV
    head h // (n_head / n_kv).  Returns [n_head][T][hd].
    """
    q, k, v = (np.asarray(a, dtype=F64) for a in (q, k, v))
    nh, T, hd = q.shape
    nkv = k.shape[0]
    group = nh // nkv
    ok = allowed_keys(q_pos, k.shape[1], window)
    out = np.empty_like(q)
    scale = hd ** -0.5
    for h in range(nh):
        g = h // group
        s = (q[h] @ k[g].T) * scale
        s = np.where(ok, s, -np.inf)
        out[h] = softmax(s) @ v[g]
    return out


def silu(x):
    x = np.asarray(x, dtype=F64)
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def gelu_erf(x):
    """Exact GELU x * Phi(x); only used to show it differs from gelu_tanh."""
    from scipy.special import erf
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


ACTS = {"silu": silu, "gelu_tanh": gelu_tanh}


def argmax_first(v):
    """Index of the largest value, the lowest index among equal maxima."""
    v = np.asarray(v)
    return int(np.argmax(v))
