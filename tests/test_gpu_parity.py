"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: dequantization, embedding gather, argmax token choice.
Within 2e-3 (max |gpu - oracle| / max |oracle| per row): projections, every
logits row of prefill and decode.  Tokens: identical wherever the oracle's
top-2 margin exceeds twice that tolerance; decode continues by teacher forcing
(the oracle consumes the GPU's tokens).
"""
import numpy as np
import pytest

import synth
from oracle import OracleModel, blocks, sampler
from tests.gpu_helpers import SMALL, TOL, as_np, check_row, rel_err, token_agrees

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import decoder_gguf_quantized_amd as qdec  # noqa: E402


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


_MODELS = {}


def model_for(key, max_ctx=256, max_seqs=2):
    """(cfg, tensors, GPU Model) cached per key."""
    if key not in _MODELS:
        cfg = synth.get(key) if key.startswith("c") else dict(SMALL[key])
        t = synth.generate(cfg)
        dev()
        _MODELS[key] = (cfg, t, qdec.Model(cfg, t, max_seqs=max_seqs, max_ctx=max_ctx))
    return _MODELS[key]


# ---------------------------------------------------------------- bit-exact pieces
@pytest.mark.parametrize("key", ["c1"] + sorted(SMALL))
def test_dequant_bit_exact(key):
    cfg, t, m = model_for(key)
    for name, tt in t.items():
        if tt.rows == 1:
            continue
        out = torch.empty((tt.rows, tt.cols), dtype=torch.float32, device=dev())
        m.debug_dequant(name, out)
        torch.cuda.synchronize()
        want = blocks.dequant(tt.type, tt.data, tt.rows, tt.cols)
        got = as_np(out)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name


@pytest.mark.parametrize("key", ["c1", "llama_q4_hd64_g4", "qwen3_hd128_g2"])
def test_embedding_gather_bit_exact(key):
    cfg, t, m = model_for(key)
    ids = np.array([0, cfg["vocab"] - 1, 7, 7, 123 % cfg["vocab"]], dtype=np.int32)
    out = torch.empty((len(ids), cfg["hidden"]), dtype=torch.float32, device=dev())
    m.debug_embed(torch.from_numpy(ids).to(dev()), out)
    torch.cuda.synchronize()
    te = t["token_embd.weight"]
    want = blocks.dequant(te.type, te.data, te.rows, te.cols)[ids]
    assert np.array_equal(as_np(out).view(np.uint32), want.view(np.uint32))


def test_argmax_bit_exact_with_ties_and_nan():
    rng = np.random.default_rng(5)
    V = 9000  # three 4096-entry chunks, ragged tail
    L = rng.standard_normal((8, V)).astype(np.float32)
    L[1, :] = 1.0                       # all equal -> 0
    L[2, 4095] = L[2, 5000] = 50.0      # tie across chunks -> 4095
    L[3, 8999] = 60.0                   # last element
    L[4, 17] = np.nan; L[4, 9] = np.nan  # first NaN wins (numpy's rule)
    L[5, :] = -np.inf; L[5, 300] = -1e30
    L[6, 4096] = np.float32(3e38)
    L[7, 0] = -0.0; L[7, 1:] = -1.0; L[7, 5] = 0.0   # -0 == +0 -> lower index
    out = torch.empty(8, dtype=torch.int32, device=dev())
    qdec.debug_sample(torch.from_numpy(L).to(dev()), 0.0, 0, 0, out)
    torch.cuda.synchronize()
    want = [sampler.greedy(r) for r in L]
    assert as_np(out).tolist() == want


def _head_rows(t, name):
    """The raw GGUF rows of a matrix as a writable [rows][row_bytes] uint8 view."""
    w = t[name]
    return w.data.reshape(w.rows, -1)


@pytest.mark.parametrize("key,case", [
    ("llama_q4_hd64_g4", "periodic"),      # Q4_0 head, four-row groups
    ("mha_hd128_g1_f32", "nan"),           # F32 head (the loader refuses non-finite block scales)
    ("qwen2_bias_hd64_g2", "periodic"),    # Q8_0 head
    ("gemma_hd256_g4", "periodic"),        # tied head, sandwich-norm prologue
])
def test_fused_greedy_choice_ties_and_nan(key, case):
    """At one row and temperature 0 the LM head's epilogue picks the token (each
    wave keeps the best of the rows it stores, then one pass over the waves):
    the token must be the greedy rule's on the GPU's own logits row, lowest
    index first among equals and the first NaN above every number.
    periodic: every head row r is a copy of row r mod 37, so the maximum is
    held by about vocab / 37 rows in many waves and the lowest one (below 37)
    must win.  nan: rows 300 and 900 of an F32 head hold a NaN; 300 must win.
    Checked through prefill's last row and through graph-replayed decode."""
    cfg = dict(SMALL[key])
    t = synth.generate(cfg)
    name = "output.weight" if "output.weight" in t else "token_embd.weight"
    rows = _head_rows(t, name)
    V = cfg["vocab"]
    if case == "periodic":
        rows[:] = rows[np.arange(V) % 37]
    else:
        rows.view(np.float32)[[300, 900], 5] = np.nan
    dev()
    # input tokens outside the changed rows' range (a tied head is the embedding)
    prompt = (synth.prompt(cfg, 6, tag="amax") % 30).astype(np.int32) + 1
    with qdec.Model(cfg, t, max_seqs=1, max_ctx=64) as m:
        pl = torch.empty(V, dtype=torch.float32, device=dev())
        tok = torch.empty(1, dtype=torch.int32, device=dev())
        m.prefill(0, prompt, pl, tok)
        torch.cuda.synchronize()
        seen = [(as_np(pl).copy(), int(as_np(tok)[0]))]
        dl = torch.empty((1, V), dtype=torch.float32, device=dev())
        out = torch.empty(1, dtype=torch.int32, device=dev())
        for step in range(3):
            m.decode_step([int(prompt[step])], dl, out)
            torch.cuda.synchronize()
            seen.append((as_np(dl)[0].copy(), int(as_np(out)[0])))
    for lg, got in seen:
        assert got == sampler.greedy(lg)
        if case == "periodic":
            # copies of a row give bit-identical logits
            assert np.array_equal(lg.view(np.uint32), lg[np.arange(V) % 37].view(np.uint32))
            assert got < 37
        else:
            assert np.isnan(lg[300]) and np.isnan(lg[900])
            assert got == 300


def test_lm_head_past_the_grid_cap():
    """A 600,000-token vocabulary: the LM head GEMV needs more than its usual
    1,024 workgroups (a wave holds at most 64 outputs), so the greedy choice
    reduces more than 8,192 per-wave partials.  Logits within the tolerance of
    the oracle's, tokens the greedy rule's on the GPU's logits, through prefill
    and replayed decode."""
    cfg = dict(SMALL["qwen3_hd128_g2"], name="wide_vocab", n_layer=1, vocab=600_000, seed=21)
    t = synth.generate(cfg)
    dev()
    V = cfg["vocab"]
    prompt = synth.prompt(cfg, 5, tag="wide")
    om = OracleModel(cfg, t, max_ctx=16)
    with qdec.Model(cfg, t, max_seqs=1, max_ctx=16) as m:
        pl = torch.empty(V, dtype=torch.float32, device=dev())
        tok = torch.empty(1, dtype=torch.int32, device=dev())
        m.prefill(0, prompt, pl, tok)
        torch.cuda.synchronize()
        g = as_np(pl).copy()
        check_row(g, om.forward(0, prompt)[0])
        assert int(as_np(tok)[0]) == sampler.greedy(g)
        dl = torch.empty((1, V), dtype=torch.float32, device=dev())
        out = torch.empty(1, dtype=torch.int32, device=dev())
        cur = int(as_np(tok)[0])
        for step in range(3):
            m.decode_step([cur], dl, out)
            torch.cuda.synchronize()
            g = as_np(dl)[0].copy()
            check_row(g, om.forward(0, [cur])[0])
            got = int(as_np(out)[0])
            assert got == sampler.greedy(g)
            cur = got


@pytest.mark.parametrize("temperature", [1.0, 0.7])
def test_gumbel_sampling_matches_oracle(temperature):
    rng = np.random.default_rng(6)
    rows, V = 16, 151936
    L = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    out = torch.empty(rows, dtype=torch.int32, device=dev())
    agree = 0
    for step in range(4):
        qdec.debug_sample(torch.from_numpy(L).to(dev()), temperature, 5, step, out)
        torch.cuda.synchronize()
        got = as_np(out)
        for r in range(rows):
            s = sampler.scores(L[r], temperature, 5, step, r)
            top2 = np.partition(s, -2)[-2:]
            if top2[1] - top2[0] > 1e-4:
                assert got[r] == int(np.argmax(s)), (step, r)
                agree += 1
    assert agree >= 60


# ---------------------------------------------------------------- top-p
def _f32(x):
    return float(np.float32(x))  # the value the library receives


@pytest.mark.parametrize("temperature,top_p,V,scale", [
    (1.0, 0.9, 151936, 3.0), (0.7, 0.5, 151936, 3.0), (1.3, 0.05, 151936, 3.0),
    # at 0.99 a 151,936-entry row's boundary sits where running sums differ by
    # ~1e-8: every row is within rounding of changing, so a smaller vocabulary
    (1.0, 0.99, 8192, 1.0),
])
def test_top_p_sampling_matches_oracle(temperature, top_p, V, scale):
    """Gumbel-max restricted to the nucleus on the same logits: the GPU token is
    the oracle's wherever the nucleus boundary is more than 1e-6 (relative) from
    changing and the top-2 perturbed scores differ by more than 1e-4; it is
    always a token the oracle's nucleus keeps, up to boundary ambiguity."""
    rng = np.random.default_rng(int(top_p * 100))
    rows = 8
    L = (rng.standard_normal((rows, V)) * scale).astype(np.float32)
    out = torch.empty(rows, dtype=torch.int32, device=dev())
    p = _f32(top_p)
    agree = 0
    for step in range(3):
        qdec.debug_sample(torch.from_numpy(L).to(dev()), temperature, 9, step, out, top_p=p)
        torch.cuda.synchronize()
        got = as_np(out)
        for r in range(rows):
            if sampler.nucleus_margin(L[r], temperature, p) <= 1e-6:
                continue
            keep = sampler.nucleus(L[r], temperature, p)
            assert keep[got[r]], (step, r)
            s = sampler.scores(L[r], temperature, 9, step, r, p)
            top2 = np.partition(s[keep], -2)[-2:] if keep.sum() > 1 else np.array([-np.inf, 0.0])
            if top2[1] - top2[0] > 1e-4:
                assert got[r] == int(np.argmax(s)), (step, r)
                agree += 1
    assert agree >= 8


@pytest.mark.parametrize("top_p,kept", [(0.5, 32), (0.3, 20), (0.25, 16), (1e-9, 1), (0.0, 1)])
def test_top_p_boundary_inside_equal_logits(top_p, kept):
    """64 equal logits (probabilities 1/64, running sums exact): the nucleus is
    the first `kept` tokens by index on both sides, so every draw is the
    oracle's and stays below index `kept`."""
    V = 64
    L = np.zeros((4, V), np.float32)
    L[1] += 2.5
    L[2] -= 7.0
    L[3, :] = -0.0
    out = torch.empty(4, dtype=torch.int32, device=dev())
    p = _f32(top_p)
    for r in range(4):
        assert sampler.nucleus(L[r], 1.0, p).sum() == kept
    for step in range(12):
        qdec.debug_sample(torch.from_numpy(L).to(dev()), 1.0, 3, step, out, top_p=p)
        torch.cuda.synchronize()
        got = as_np(out).tolist()
        want = [sampler.sample(L[r], 1.0, 3, step, r, p) for r in range(4)]
        assert got == want, (step, got, want)
        assert max(got) < kept


def test_top_p_mixed_rows_and_limits():
    """A peaked row (small nucleus), ties straddling the boundary after a run of
    distinct values, a row with NaN (every token kept: the first NaN wins), and
    top_p >= 1 (plain Gumbel-max)."""
    V = 5000
    rng = np.random.default_rng(12)
    L = (rng.standard_normal((3, V)) * 0.5).astype(np.float32)
    L[0, 123] = 9.0; L[0, 4000] = 8.5; L[0, 77] = 8.0
    L[1, :40] = 6.0; L[1, 40:] = -30.0; L[1, 3] = 6.5     # boundary inside the 6.0 run
    L[2, 17] = np.nan
    out = torch.empty(3, dtype=torch.int32, device=dev())
    for top_p in (0.6, 0.95, 1.0):
        p = _f32(top_p)
        for step in range(6):
            qdec.debug_sample(torch.from_numpy(L).to(dev()), 1.0, 21, step, out, top_p=p)
            torch.cuda.synchronize()
            got = as_np(out).tolist()
            want = [sampler.sample(L[r], 1.0, 21, step, r, p) for r in range(3)]
            assert got == want, (top_p, step, got, want)


def test_top_p_nan_is_refused():
    L = torch.zeros((1, 10), dtype=torch.float32, device=dev())
    out = torch.empty(1, dtype=torch.int32, device=dev())
    with pytest.raises(qdec.QdecError):
        qdec.debug_sample(L, 1.0, 0, 0, out, top_p=float("nan"))


# ---------------------------------------------------------------- projections
MATMUL_CASES = [
    # (type, rows, cols, n_x)
    (synth.T_Q8_0, 4096, 1024, 1), (synth.T_Q8_0, 1000, 688, 3), (synth.T_Q8_0, 257, 1152, 16),
    (synth.T_Q8_0, 300, 256, 17), (synth.T_Q8_0, 1024, 3072, 130),
    (synth.T_Q4_0, 6144, 4096, 1), (synth.T_Q4_0, 130, 14336, 2), (synth.T_Q4_0, 512, 1408, 9),
    (synth.T_Q4_0, 333, 512, 70),
    (synth.T_F32, 1024, 256, 1), (synth.T_F32, 200, 352, 5), (synth.T_F32, 129, 96, 65),
    # prefill tiles: >= 512 tiles of 64 x 128 (ragged rows and tokens) take the
    # wide tile; fewer take the K-split 32 x 64 tile (partial last K stage)
    (synth.T_Q8_0, 4100, 320, 1030), (synth.T_Q4_0, 4224, 288, 1000),
    # Q4_0 / Q8_0 wide tiles stage block pairs: an odd block count leaves the
    # last stage half empty (Q4_0 above: 9 blocks; Q8_0 here: 11)
    (synth.T_Q8_0, 4100, 352, 1000),
    (synth.T_Q4_0, 200, 720, 40), (synth.T_F32, 96, 300, 33), (synth.T_Q8_0, 1030, 1000, 97),
    # one input row, >= 4,096 rows of >= 8,192 inputs: sixteen-wave workgroups
    # of one row per wave (ragged rows; Q4_0 in the next group)
    (synth.T_Q8_0, 4097, 9216, 1), (synth.T_Q4_K, 4100, 8448, 1), (synth.T_Q6_K, 4099, 8192, 1),
    (synth.T_F32, 4096, 8192, 1),
    # 5..16 input rows, >= 2,048 outputs: the matrix-core decode (ragged rows,
    # block counts that are not multiples of four)
    (synth.T_Q8_0, 2100, 1024, 16), (synth.T_Q4_0, 4100, 1120, 9), (synth.T_Q8_0, 2048, 4128, 12),
    (synth.T_Q4_0, 3000, 2080, 13), (synth.T_Q8_0, 2050, 1056, 5), (synth.T_Q4_0, 2060, 1024, 8),
    (synth.T_Q4_K, 2100, 1280, 12), (synth.T_Q6_K, 2060, 2048, 7), (synth.T_Q6_K, 4097, 768, 16),
    # long rows with >= 2048 row groups: eight-wave workgroups (ragged rows)
    (synth.T_Q4_0, 4100, 8192, 1), (synth.T_Q4_0, 4097, 4608, 2), (synth.T_Q8_0, 4100, 2080, 3),
    (synth.T_F32, 4100, 600, 5),
    # K-quants (repacked to 32-value blocks with f32 scales): every GEMV tile
    # class, the eight-wave class, staged input rows above 64 KB of LDS, both
    # GEMM tiles
    (synth.T_Q4_K, 4096, 1024, 1), (synth.T_Q4_K, 1000, 2816, 3), (synth.T_Q4_K, 4100, 4608, 2),
    (synth.T_Q4_K, 300, 512, 17), (synth.T_Q4_K, 4224, 256, 1000),
    (synth.T_Q6_K, 4096, 1024, 1), (synth.T_Q6_K, 257, 1536, 16), (synth.T_Q6_K, 130, 14336, 2),
    (synth.T_Q6_K, 4100, 2048, 3), (synth.T_Q6_K, 1030, 1024, 97), (synth.T_Q6_K, 4100, 512, 1030),
    # 256..511 tiles of 64 x 128: the f32 path takes the K-split tile, the bf16
    # paths the wide bf16 tile
    (synth.T_Q8_0, 2048, 512, 1000), (synth.T_Q4_0, 2304, 288, 900),
    # input rows beyond the 128 KB LDS budget of one launch: two 8-row launches,
    # and three launches of 2, 2 and 1 rows
    (synth.T_Q8_0, 300, 4096, 16), (synth.T_Q4_0, 100, 14336, 5),
]


@pytest.mark.parametrize("ttype,rows,cols,n_x", MATMUL_CASES)
def test_projection_matches_oracle(ttype, rows, cols, n_x):
    rng = np.random.default_rng(rows * 7 + cols + n_x)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    raw = synth.encode(ttype, w)
    kp = ((cols + 31) // 32) * 32
    x = np.zeros((n_x, kp), np.float32)
    x[:, :cols] = rng.standard_normal((n_x, cols))
    y = torch.empty((n_x, rows), dtype=torch.float32, device=dev())
    qdec.debug_matmul(ttype, rows, cols, raw, torch.from_numpy(x).to(dev()), y)
    W = blocks.dequant(ttype, raw, rows, cols).astype(np.float64)
    want = x[:, :cols].astype(np.float64) @ W.T
    got = as_np(y)
    for r in range(n_x):
        check_row(got[r], want[r])


GEMM_CASES = [c for c in MATMUL_CASES if c[3] > 16 and c[0] in (synth.T_Q8_0, synth.T_Q4_0)]


def one_hot_columns(cols, n_x):
    """Columns k_t picked by input row t: the first and last column, block
    edges and a spread over the row, cycling when n_x exceeds them."""
    base = sorted({0, cols - 1, min(31, cols - 1), min(32, cols - 1), cols // 2, max(0, cols - 33)})
    spread = [(t * 7919) % cols for t in range(n_x)]
    return [(base + spread)[t] for t in range(n_x)]


@pytest.mark.parametrize("precision", ["f32", "bf16x3"])
@pytest.mark.parametrize("ttype,rows,cols,n_x", MATMUL_CASES)
def test_projection_kernels_decode_weights_bit_exact(ttype, rows, cols, n_x, precision):
    """The projection kernels themselves decode every weight exactly: with input
    row t one-hot at column k_t, output (t, n) is the single product W[n][k_t] * 1
    plus exact zeros, so it must equal the oracle's exact dequantisation bit for
    bit (up to the sign of zero) -- through each GEMV tile class (n_x <= 16), the
    wide and K-split f32 GEMM tiles and the three-term bf16 tile."""
    if precision == "bf16x3" and (n_x <= 16 or ttype not in (synth.T_Q8_0, synth.T_Q4_0)):
        pytest.skip("the bf16 tile serves Q8_0 / Q4_0 prefill projections only")
    rng = np.random.default_rng(rows * 3 + cols + n_x)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    raw = synth.encode(ttype, w)
    kp = ((cols + 31) // 32) * 32
    ks = one_hot_columns(cols, n_x)
    x = np.zeros((n_x, kp), np.float32)
    x[np.arange(n_x), ks] = 1.0
    y = torch.empty((n_x, rows), dtype=torch.float32, device=dev())
    qdec.debug_matmul(ttype, rows, cols, raw, torch.from_numpy(x).to(dev()), y, precision=precision)
    W = blocks.dequant(ttype, raw, rows, cols)
    want = W[:, ks].T
    got = as_np(y)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {tuple(bad[0])}: {got[tuple(bad[0])]!r} vs {want[tuple(bad[0])]!r}"


@pytest.mark.parametrize("ttype,rows,cols,n_x", GEMM_CASES)
def test_projection_bf16x3_matches_oracle(ttype, rows, cols, n_x):
    """The three-term bf16 split is exact: same bar as the f32 kernels, and in
    practice f32-level agreement (max relative error per row below 1e-5)."""
    rng = np.random.default_rng(rows * 7 + cols + n_x)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    raw = synth.encode(ttype, w)
    kp = ((cols + 31) // 32) * 32
    x = np.zeros((n_x, kp), np.float32)
    x[:, :cols] = rng.standard_normal((n_x, cols))
    y = torch.empty((n_x, rows), dtype=torch.float32, device=dev())
    qdec.debug_matmul(ttype, rows, cols, raw, torch.from_numpy(x).to(dev()), y, precision="bf16x3")
    W = blocks.dequant(ttype, raw, rows, cols).astype(np.float64)
    want = x[:, :cols].astype(np.float64) @ W.T
    got = as_np(y)
    errs = [check_row(got[r], want[r]) for r in range(n_x)]
    assert max(errs) < 1e-5, max(errs)


def test_projection_bf16_plain_error_is_reported():
    """Activations rounded to bf16 (one term): the error is bf16's (about 2^-9
    per product, averaging down over K); it is measured, not held to 2e-3.
    (The shape fills >= 512 wide tiles, so the bf16 kernel runs.)"""
    rng = np.random.default_rng(44)
    rows, cols, n_x = 4096, 512, 1024
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    raw = synth.encode(synth.T_Q8_0, w)
    x = rng.standard_normal((n_x, cols)).astype(np.float32)
    y = torch.empty((n_x, rows), dtype=torch.float32, device=dev())
    qdec.debug_matmul(synth.T_Q8_0, rows, cols, raw, torch.from_numpy(x).to(dev()), y, precision="bf16")
    W = blocks.dequant(synth.T_Q8_0, raw, rows, cols).astype(np.float64)
    want = x.astype(np.float64) @ W.T
    got = as_np(y)
    err = max(float(np.max(np.abs(got[r] - want[r])) / np.max(np.abs(want[r]))) for r in range(n_x))
    print(f"plain bf16 activations: max relative error per row {err:.2e}")
    assert 1e-5 < err < 2e-2


# ---------------------------------------------------------------- whole model
def run_gpu(m, cfg, prompt, n_steps, seq=0):
    """Prefill (all logits) then n_steps greedy decode steps chained on device.
    Returns prefill logits [T][V], decode logits [n][V], decode tokens [n]."""
    V = cfg["vocab"]
    T = len(prompt)
    pl = torch.empty((T, V), dtype=torch.float32, device=dev())
    tok = torch.empty(1, dtype=torch.int32, device=dev())
    m.kv_reset()
    m.prefill(seq, prompt, pl, tok, all_logits=True)
    dl = torch.empty((n_steps, V), dtype=torch.float32, device=dev())
    toks = torch.empty((n_steps, 1), dtype=torch.int32, device=dev())
    cur = tok
    for s in range(n_steps):
        m.decode_step(cur, dl[s:s + 1], toks[s])
        cur = toks[s]
    torch.cuda.synchronize()
    first = int(as_np(tok)[0])
    return as_np(pl), as_np(dl), [first] + as_np(toks).reshape(-1).tolist()


def oracle_run(cfg, t, prompt, gpu_tokens, n_steps):
    om = OracleModel(cfg, t, max_ctx=len(prompt) + n_steps + 1)
    pl = om.forward(0, prompt, all_logits=True)
    dl = [om.forward(0, [gpu_tokens[s]])[0] for s in range(n_steps)]
    return pl, np.array(dl)


@pytest.mark.parametrize("key", ["c1"] + sorted(SMALL))
def test_prefill_and_decode_match_oracle(key):
    cfg, t, m = model_for(key)
    T, n = 70, 12
    prompt = synth.prompt(cfg, T)
    g_pl, g_dl, g_tok = run_gpu(m, cfg, prompt, n)
    o_pl, o_dl = oracle_run(cfg, t, prompt, g_tok, n)
    errs = [check_row(g_pl[i], o_pl[i]) for i in range(T)]
    errs += [check_row(g_dl[s], o_dl[s]) for s in range(n)]
    assert token_agrees(g_tok[0], o_pl[-1])
    for s in range(n):
        assert token_agrees(g_tok[s + 1], o_dl[s])
    print(f"{key}: max rel err {max(errs):.2e}")


@pytest.mark.parametrize("key", ["llama_q4_hd64_g4", "qwen3_hd128_g2", "gemma_hd256_g4"])
def test_bf16x3_prefill_matches_oracle(key):
    """Prefill with the three-term bf16 split in every quantized projection:
    every position's logits within the f32 path's tolerance."""
    cfg, t, m = model_for(key)
    T = 70
    prompt = synth.prompt(cfg, T)
    m.set_prefill_precision("bf16x3")
    try:
        g_pl, _, g_tok = run_gpu(m, cfg, prompt, 0)
    finally:
        m.set_prefill_precision("f32")
    o_pl, _ = oracle_run(cfg, t, prompt, g_tok, 0)
    errs = [check_row(g_pl[i], o_pl[i]) for i in range(T)]
    assert token_agrees(g_tok[0], o_pl[-1])
    print(f"{key} bf16x3: max rel err {max(errs):.2e}")


@pytest.mark.parametrize("key", ["c1", "gemma_hd256_g4"])
def test_gpu_decode_equals_gpu_prefill_recompute(key):
    cfg, t, m = model_for(key)
    prompt = synth.prompt(cfg, 20)
    g_pl, g_dl, g_tok = run_gpu(m, cfg, prompt, 6)
    full = list(prompt) + g_tok[:6]
    V = cfg["vocab"]
    pl = torch.empty((len(full), V), dtype=torch.float32, device=dev())
    m.kv_reset()
    m.prefill(0, full, pl, None, all_logits=True)
    torch.cuda.synchronize()
    rec = as_np(pl)
    for s in range(6):
        check_row(g_dl[s], rec[20 + s])


def test_window_ring_matches_the_full_cache():
    """Window layers' rings ([P] roadmap table: a paged or ring-buffer cache)
    give the results of caches that keep every position: a prompt longer than
    the ring (three prefill passes, wrapped slots) bit for bit, decode steps
    past it to f32 rounding (the merge's adds vary in order), and preset
    positions written past the ring's length."""
    cfg, t, _ = model_for("gemma_hd256_g4")
    V, L = cfg["vocab"], cfg["n_layer"]
    # window 8, passes of 4,096 positions: rings of 8,192 positions
    prompt = synth.prompt(cfg, 9000, tag="ring")
    follow = synth.prompt(cfg, 24, tag="ring-next")
    with qdec.Model(cfg, t, max_seqs=1, max_ctx=16384) as m:
        rings = [m.kv_ring_positions(l) for l in range(L)]
        assert sorted(set(rings)) == [0, 8192], rings  # global layers keep every position
        last = list(range(len(prompt) - 40, len(prompt)))  # prefill rows compared

        def run():
            pl = torch.empty((len(prompt), V), dtype=torch.float32, device=dev())
            dl = torch.empty((len(follow), V), dtype=torch.float32, device=dev())
            tk = torch.empty(1, dtype=torch.int32, device=dev())
            m.kv_reset()
            m.prefill(0, prompt, pl, None, all_logits=True)
            for s, tok in enumerate(follow):  # the same host tokens on both layouts
                m.decode_step([tok], dl[s:s + 1], tk)
            torch.cuda.synchronize()
            return as_np(pl[last]), as_np(dl)

        ring_pl, ring_dl = run()
        with pytest.raises(qdec.QdecError):
            m.kv_ring(False)  # sequence 0 holds positions
        m.kv_reset()
        m.kv_ring(False)
        assert [m.kv_ring_positions(l) for l in range(L)] == [0] * L
        full_pl, full_dl = run()
        assert np.array_equal(ring_pl, full_pl)
        for s in range(len(follow)):
            check_row(ring_dl[s], full_dl[s], tol=1e-5)

        # preset positions: 8,392 per layer (the ring keeps the last 8,192),
        # written on both layouts, then one step
        n_pos = 8192 + 200
        rng = np.random.default_rng(5)
        shape = (cfg["n_head_kv"], n_pos, cfg["head_dim"])
        kv = [(torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dev()),
               torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dev())) for _ in range(L)]
        out = {}
        for ring in (False, True):
            m.kv_reset()
            m.kv_ring(ring)
            for l in range(L):
                m.kv_write(0, l, *kv[l])
            row = torch.empty((1, V), dtype=torch.float32, device=dev())
            m.decode_step([follow[0]], row, torch.empty(1, dtype=torch.int32, device=dev()))
            torch.cuda.synchronize()
            out[ring] = as_np(row)[0]
        check_row(out[True], out[False], tol=1e-5)

        # truncation keeps the window whole only within R - window positions
        n = n_pos + 1
        with pytest.raises(qdec.QdecError):
            m.kv_truncate(0, n - (8192 - 8) - 1)
        m.kv_truncate(0, n - (8192 - 8))
        assert m.kv_len(0) == n - (8192 - 8)


def test_split_prefill_and_reset_are_consistent():
    cfg, t, m = model_for("qwen3_hd128_g2")
    V = cfg["vocab"]
    prompt = synth.prompt(cfg, 90)
    a = torch.empty(V, dtype=torch.float32, device=dev())
    b = torch.empty(V, dtype=torch.float32, device=dev())
    c = torch.empty(V, dtype=torch.float32, device=dev())
    m.kv_reset()
    m.prefill(0, prompt, a)
    m.kv_reset()
    m.prefill(0, prompt[:37], b)
    m.prefill(0, prompt[37:], b)
    m.kv_reset()
    m.prefill(0, prompt, c)
    torch.cuda.synchronize()
    check_row(as_np(b), as_np(a))
    assert np.array_equal(as_np(a), as_np(c))  # reset then rerun: bit-identical
    assert m.kv_len(0) == 90


def test_two_sequences_are_independent():
    cfg, t, m = model_for("qwen3_hd128_g2")
    V = cfg["vocab"]
    p0, p1 = synth.prompt(cfg, 30), synth.prompt(cfg, 45, tag="other")
    l0 = torch.empty(V, dtype=torch.float32, device=dev())
    l1 = torch.empty(V, dtype=torch.float32, device=dev())
    m.kv_reset()
    m.prefill(0, p0, l0)
    m.prefill(1, p1, l1)
    dl = torch.empty((2, V), dtype=torch.float32, device=dev())
    tk = torch.empty(2, dtype=torch.int32, device=dev())
    m.decode_step([5, 9], dl, tk)
    torch.cuda.synchronize()
    om = OracleModel(cfg, t, max_ctx=64, n_seqs=2)
    om.forward(0, p0)
    om.forward(1, p1)
    o = om.decode([5, 9])
    check_row(as_np(dl)[0], o[0])
    check_row(as_np(dl)[1], o[1])
    assert m.kv_len(0) == 31 and m.kv_len(1) == 46


def test_decode_step_top_p_follows_the_oracle_sampler():
    """Two sequences, temperature 0.8 with top_p 0.9, tokens fed back on the
    device: each step's logits match the oracle (teacher forced) and each
    sampled token is the oracle sampler's on the GPU's logits wherever the
    nucleus boundary and the top-2 perturbed scores are clear.  Greedy steps in
    between use the graph without the top-p cut; a top_p >= 1 step equals plain
    Gumbel-max."""
    cfg, t, m = model_for("qwen3_hd128_g2")
    V = cfg["vocab"]
    p0, p1 = synth.prompt(cfg, 20), synth.prompt(cfg, 33, tag="other")
    lg = torch.empty(V, dtype=torch.float32, device=dev())
    m.kv_reset()
    m.prefill(0, p0, lg)
    m.prefill(1, p1, lg)
    om = OracleModel(cfg, t, max_ctx=64, n_seqs=2)
    om.forward(0, p0)
    om.forward(1, p1)
    T, P = 0.8, _f32(0.9)
    toks = torch.tensor([3, 7], dtype=torch.int32, device=dev())
    plan = [(T, P), (T, P), (0.0, 1.0), (T, P), (T, 1.0), (T, P)]
    checked = 0
    for step, (temp, top_p) in enumerate(plan):
        inp = as_np(toks).tolist()
        dl = torch.empty((2, V), dtype=torch.float32, device=dev())
        out = torch.empty(2, dtype=torch.int32, device=dev())
        m.decode_step(toks, dl, out, temperature=temp, seed=77, step=step, top_p=top_p)
        torch.cuda.synchronize()
        g = as_np(dl)
        o = om.decode(inp)
        got = as_np(out).tolist()
        for sq in range(2):
            check_row(g[sq], o[sq])
            if temp == 0.0:
                assert got[sq] == sampler.greedy(g[sq])
                continue
            if sampler.nucleus_margin(g[sq], temp, top_p) <= 1e-6:
                continue
            sc = sampler.scores(g[sq], temp, 77, step, sq, top_p)
            top2 = np.partition(sc, -2)[-2:]
            if top2[1] - top2[0] > 1e-4:
                assert got[sq] == int(np.argmax(sc)), (step, sq)
                checked += 1
        toks = out
    assert checked >= 8


def test_decode_ignores_cache_rows_past_the_length():
    """Cache rows past a sequence's length hold NaN (written, then truncated
    away); decode attention requests whole chunks ahead of the position, so it
    reads them, and must mask them without letting 0 * NaN through."""
    cfg, t, m = model_for("qwen3_hd128_g2")
    V, nkv, hd = cfg["vocab"], cfg["n_head_kv"], cfg["head_dim"]
    keep, n_pos = 60, 100
    rng = np.random.default_rng(31)
    om = OracleModel(cfg, t, max_ctx=128, n_seqs=1)
    m.kv_reset()
    for layer in range(cfg["n_layer"]):
        k = rng.standard_normal((nkv, n_pos, hd)).astype(np.float32)
        v = rng.standard_normal((nkv, n_pos, hd)).astype(np.float32)
        om.kv_write(0, layer, k[:, :keep], v[:, :keep])
        k[:, keep:] = np.nan
        v[:, keep:] = np.nan
        m.kv_write(0, layer, torch.from_numpy(k).to(dev()), torch.from_numpy(v).to(dev()))
    m.kv_truncate(0, keep)
    om.set_kv_len(0, keep)
    dl = torch.empty((1, V), dtype=torch.float32, device=dev())
    out = torch.empty(1, dtype=torch.int32, device=dev())
    for step, tok in enumerate([11, 29, 7]):
        m.decode_step([tok], dl, out)
        torch.cuda.synchronize()
        check_row(as_np(dl)[0], om.forward(0, [tok])[0])


@pytest.mark.parametrize("key", ["llama_q4_hd64_g4", "qwen3_hd128_g2", "gemma_hd256_g4"])
def test_prefill_ignores_cache_rows_past_the_prompt(key):
    """Prefill attention reads the last key tile of a query tile whole: the rows
    past the prompt's last key (here NaN, written and then truncated away) read
    as zeros through the tile's buffer descriptor and are masked, so the logits
    equal those over a clean cache bit for bit (head_dim 64, 128 and 256)."""
    cfg, t, m = model_for(key)
    V, nkv, hd, L = cfg["vocab"], cfg["n_head_kv"], cfg["head_dim"], cfg["n_layer"]
    prompt = synth.prompt(cfg, 70, tag="past-the-prompt")  # last tile: keys 64..95, 26 rows past key 69

    def prefill():
        pl = torch.empty((len(prompt), V), dtype=torch.float32, device=dev())
        m.prefill(0, prompt, pl, None, all_logits=True)
        torch.cuda.synchronize()
        return as_np(pl)

    m.kv_reset()
    clean = prefill()
    nan = torch.full((nkv, 200, hd), float("nan"), dtype=torch.float32, device=dev())
    m.kv_reset()
    for layer in range(L):
        m.kv_write(0, layer, nan, nan)
    m.kv_truncate(0, 0)
    dirty = prefill()
    assert np.isfinite(dirty).all()
    assert np.array_equal(clean, dirty)


@pytest.mark.parametrize("key", ["qwen3_hd128_g2", "gemma_hd256_g4"])
def test_one_token_prompt_and_a_full_cache(key):
    """The degenerate lengths: a one-token prompt (one query, one key), then
    decode up to exactly max_ctx positions, each row against the oracle; one
    step more is refused before anything is enqueued, and the handle stays
    usable."""
    cfg, t, _ = model_for(key)
    V, max_ctx = cfg["vocab"], 40
    with qdec.Model(cfg, t, max_seqs=1, max_ctx=max_ctx) as m:
        prompt = synth.prompt(cfg, 1, tag="one")
        g_pl, g_dl, g_tok = run_gpu(m, cfg, prompt, max_ctx - 1)
        o_pl, o_dl = oracle_run(cfg, t, prompt, g_tok, max_ctx - 1)
        check_row(g_pl[0], o_pl[0])
        for s in range(max_ctx - 1):
            check_row(g_dl[s], o_dl[s])
        assert m.kv_len(0) == max_ctx
        lg = torch.empty((1, V), dtype=torch.float32, device=dev())
        with pytest.raises(qdec.QdecError):
            m.decode_step([1], lg, torch.empty(1, dtype=torch.int32, device=dev()))
        with pytest.raises(qdec.QdecError):
            m.prefill(0, [1], lg[0])
        assert not m.poisoned and m.kv_len(0) == max_ctx


def test_refusals_leave_handle_usable():
    cfg, t, m = model_for("c1")
    V = cfg["vocab"]
    lg = torch.empty(V, dtype=torch.float32, device=dev())
    with pytest.raises(qdec.QdecError):
        m.prefill(0, [V], lg)
    with pytest.raises(qdec.QdecError):
        m.prefill(5, [1], lg)
    with pytest.raises(qdec.QdecError):
        m.decode_step([1], lg, torch.empty(1, dtype=torch.int32, device=dev()), temperature=-1.0)
    m.kv_reset()
    m.prefill(0, [1, 2, 3], lg)
    assert not m.poisoned and m.kv_len(0) == 3
