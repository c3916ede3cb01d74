"""Token choice: greedy argmax and temperature sampling by Gumbel-max.

Greedy follows the walkthrough's Step 8 (temperature 0 -> argmax of the
logits); ties go to the lowest index, and NaN ranks above every number (numpy's
argmax rule).  Temperature T > 0 draws from softmax(logits / T) (Step 8).  The
draw is taken as argmax_v(logits_v / T + G_v) with Gumbel noise
G_v = -ln(-ln u_v), which samples exactly that distribution and needs no
ordered prefix sum.  The uniforms come from Philox4x64-10 (Salmon, Moraes, Dror,
Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11), a counter-based
generator:

  counter = (v // 4, step, seq, 0), key = (seed, 0), word = v % 4
  u_v = ((r >> 41) + 0.5) * 2^-23        (top 23 bits; exact in float32 and
                                          strictly inside (0, 1), so G is finite)

Top-p (nucleus) sampling follows the walkthrough's Step 8 sampler: with
probabilities p = softmax(logits / T), sort them in descending order, take the
running sum, keep the first count(running sum < top_p) + 1 tokens (the smallest
prefix whose mass reaches top_p), renormalise and draw.  Readings: equal
probabilities are ordered by lower index first (a stable sort); top_p >= 1, or
a row with a NaN or infinite logit, keeps every token.  The draw over the kept
set is the same Gumbel-max (renormalising shifts every kept log-probability by
one constant, which leaves the argmax unchanged).

Philox4x64-10: ten rounds of
  (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2          (128-bit products)
  c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
with the key bumped by the Weyl constants (W0, W1) between rounds; M0, M1, W0,
W1 are the paper's 64-bit multipliers and Weyl increments.
"""
import numpy as np

U64 = np.uint64
M32 = U64(0xFFFFFFFF)
PHILOX_M0 = U64(0xD2E7470EE14C6C93)
PHILOX_M1 = U64(0xCA5A826395121157)
PHILOX_W0 = U64(0x9E3779B97F4A7C15)
PHILOX_W1 = U64(0xBB67AE8584CAA73B)


def _mulhilo(a, b):
    """128-bit product of uint64 arrays: (high 64 bits, low 64 bits)."""
    a = np.asarray(a, U64)
    b = np.asarray(b, U64)
    alo, ahi = a & M32, a >> U64(32)
    blo, bhi = b & M32, b >> U64(32)
    p0 = alo * blo
    p1 = alo * bhi
    p2 = ahi * blo
    p3 = ahi * bhi
    mid = (p0 >> U64(32)) + (p1 & M32) + (p2 & M32)
    hi = p3 + (p1 >> U64(32)) + (p2 >> U64(32)) + (mid >> U64(32))
    lo = a * b
    return hi, lo


def philox4x64_10(ctr, key):
    """ctr: 4 uint64 arrays (broadcastable), key: 2 uint64 values -> 4 uint64 arrays."""
    with np.errstate(over="ignore"):
        c0, c1, c2, c3 = (np.asarray(c, U64) for c in ctr)
        k0, k1 = U64(key[0]), U64(key[1])
        for r in range(10):
            if r:
                k0 = U64(k0 + PHILOX_W0)
                k1 = U64(k1 + PHILOX_W1)
            hi0, lo0 = _mulhilo(PHILOX_M0, c0)
            hi1, lo1 = _mulhilo(PHILOX_M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniforms(vocab, seed, step, seq):
    """u_v for v in [0, vocab) as float32, per the counter layout above."""
    v = np.arange(vocab, dtype=np.uint64)
    words = philox4x64_10((v >> U64(2), U64(step), U64(seq), U64(0)), (seed & 0xFFFFFFFFFFFFFFFF, 0))
    w = np.stack(words, axis=0)
    r = w[(v & U64(3)).astype(np.int64), np.arange(vocab)]
    return (((r >> U64(41)).astype(np.float64) + 0.5) * 2.0 ** -23).astype(np.float32)


def gumbel(vocab, seed, step, seq):
    """G_v = -ln(-ln u_v), float64 from the float32 uniform."""
    u = uniforms(vocab, seed, step, seq).astype(np.float64)
    return -np.log(-np.log(u))


def greedy(logits):
    """argmax with the lowest index on ties (NaN ranks above every number)."""
    return int(np.argmax(np.asarray(logits)))


def nucleus_from_probs(probs, top_p):
    """Boolean mask of the tokens top-p keeps, from probabilities (float64):
    descending order with ties by lower index, running sum, the first
    count(running sum < top_p) + 1 tokens."""
    p = np.asarray(probs, dtype=np.float64)
    order = np.argsort(-p, kind="stable")
    run = np.cumsum(p[order])
    cutoff = int(np.sum(run < top_p)) + 1
    keep = np.zeros(p.size, dtype=bool)
    keep[order[:cutoff]] = True
    return keep


def softmax_t(logits, temperature):
    """softmax(logits / T) in float64."""
    z = np.asarray(logits, dtype=np.float64) / temperature
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def nucleus(logits, temperature, top_p):
    """Mask of the tokens top-p keeps for one row (every token for top_p >= 1,
    temperature 0, or a row with a non-finite logit)."""
    lg = np.asarray(logits, dtype=np.float64)
    if top_p >= 1 or temperature == 0 or not np.all(np.isfinite(lg)):
        return np.ones(lg.size, dtype=bool)
    return nucleus_from_probs(softmax_t(lg, temperature), top_p)


def nucleus_margin(logits, temperature, top_p):
    """How far the kept set is from changing under rounding of the running
    sums: the smaller of |run - top_p| / top_p at the last kept and the first
    dropped running sum (infinity when every token is kept by rule).  The order
    itself cannot change: for T > 0 it is the order of the given logits, which
    any implementation sees exactly."""
    lg = np.asarray(logits, dtype=np.float64)
    if top_p >= 1 or temperature == 0 or not np.all(np.isfinite(lg)):
        return np.inf
    p = softmax_t(lg, temperature)
    run = np.cumsum(p[np.argsort(-p, kind="stable")])
    c = int(np.sum(run < top_p)) + 1
    m = np.inf
    for k in (c - 2, c - 1):
        if 0 <= k < run.size:
            m = min(m, abs(run[k] - top_p) / top_p)
    return m


def sample(logits, temperature, seed, step, seq, top_p=1.0):
    """Greedy for temperature 0, else argmax(logits / T + Gumbel) over the
    tokens top-p keeps."""
    if temperature == 0:
        return greedy(logits)
    return int(np.argmax(scores(logits, temperature, seed, step, seq, top_p)))


def scores(logits, temperature, seed, step, seq, top_p=1.0):
    """The perturbed scores the sampler takes the argmax of (-inf outside the
    kept set)."""
    lg = np.asarray(logits, dtype=np.float64)
    if temperature == 0:
        return lg
    sc = lg / temperature + gumbel(lg.size, seed, step, seq)
    keep = nucleus(lg, temperature, top_p)
    return np.where(keep, sc, -np.inf)


def uniforms_batch(vocab, seed, steps, seq):
    """u[step][v] for many steps at once (same layout as ``uniforms``)."""
    steps = np.asarray(steps, dtype=np.uint64)[:, None]
    v = np.arange(vocab, dtype=np.uint64)[None, :]
    words = philox4x64_10((v >> U64(2), steps, U64(seq), U64(0)), (seed & 0xFFFFFFFFFFFFFFFF, 0))
    w = np.stack(np.broadcast_arrays(*words), axis=0)
    sel = np.broadcast_to((v & U64(3)).astype(np.int64), w.shape[1:])
    r = np.take_along_axis(w, sel[None], axis=0)[0]
    return (((r >> U64(41)).astype(np.float64) + 0.5) * 2.0 ** -23).astype(np.float32)
