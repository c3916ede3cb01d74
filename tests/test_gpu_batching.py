"""GPU parity of continuous batching (qdec_decode_batch) and the paged KV cache
(qdec_kv_paged), through the C ABI.

- A schedule of arrivals (prefill into a free slot), departures (kv_reset), a
  rollback (kv_truncate) and decode steps over changing sets of slots in a
  shuffled row order: every logits row within 2e-3 of the oracle, which runs
  each slot as its own sequence; greedy tokens as in the other parity tests,
  fed back by teacher forcing.
- The same schedule on a paged cache (pages recycled between sequences) and
  on the contiguous cache: the same logits up to f32 rounding (the paging changes addresses
  only; the page size equals the decode chunk, so the split is the same).
- A sliding-window model whose prefill tiles straddle pages.
- Sampled decode of a slot: the token is the oracle sampler's on the GPU's own
  logits with the slot as the stream's sequence index.
- Refusals: an exhausted pool, a cache in use, bad page sizes, repeated or
  out-of-range slots; the handle stays usable after each.
"""
import numpy as np
import pytest

import synth
from oracle import OracleModel, sampler
from tests.gpu_helpers import SMALL, as_np, check_row, rel_err, token_agrees

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import decoder_gguf_quantized_amd as qdec  # noqa: E402


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


# (step, event, slot, argument): prefill a prompt of `argument` tokens into a
# free slot, reset a slot, truncate a slot to `argument` positions
EVENTS = [(0, "prefill", 0, 70), (0, "prefill", 2, 5), (0, "prefill", 3, 130),
          (5, "prefill", 1, 40), (10, "reset", 2, 0), (12, "truncate", 3, 64),
          (15, "prefill", 2, 100), (22, "reset", 0, 0), (24, "prefill", 0, 9)]
STEPS = 30


def run_schedule(m, cfg, om=None, pages=None):
    """Drive the schedule on GPU model m (and the oracle om, if given).
    Returns every decode logits row keyed by (step, slot)."""
    V = cfg["vocab"]
    rng = np.random.default_rng(5)
    live = {}
    rows = {}
    pl = torch.empty((256, V), dtype=torch.float32, device=dev())
    tok = torch.empty(1, dtype=torch.int32, device=dev())
    dl = torch.empty((4, V), dtype=torch.float32, device=dev())
    out = torch.empty(4, dtype=torch.int32, device=dev())
    m.kv_reset()
    if om is not None:
        om.reset()
    for step in range(STEPS):
        for (st, ev, slot, arg) in EVENTS:
            if st != step:
                continue
            if ev == "prefill":
                prompt = synth.prompt(cfg, arg, tag=f"p{step}.{slot}")
                m.prefill(slot, prompt, pl[:1], tok)
                torch.cuda.synchronize()
                live[slot] = int(as_np(tok)[0])
                if om is not None:
                    o = om.forward(slot, prompt)[0]
                    check_row(as_np(pl[0]), o)
                    assert token_agrees(live[slot], o)
            elif ev == "reset":
                m.kv_reset(slot)
                live.pop(slot)
                if om is not None:
                    om.reset(slot)
            else:
                m.kv_truncate(slot, arg)
                if om is not None:
                    om.set_kv_len(slot, arg)
        if pages is not None:
            ps, n_pages, n_free = m.kv_pages()
            held = sum(-(-m.kv_len(s) // ps) for s in range(4))
            assert n_free == n_pages - held, (step, n_free, held)
        seqs = sorted(live)
        rng.shuffle(seqs)
        n = len(seqs)
        m.decode_batch(seqs, [live[s] for s in seqs], dl[:n], out[:n])
        torch.cuda.synchronize()
        g = as_np(dl[:n]).copy()
        got = as_np(out[:n]).tolist()
        for r, s in enumerate(seqs):
            rows[(step, s)] = g[r]
            if om is not None:
                o = om.forward(s, [live[s]])[0]
                check_row(g[r], o)
                assert token_agrees(got[r], o), (step, s)
            live[s] = got[r]
    return rows


@pytest.fixture(scope="module")
def qwen3_pair():
    cfg = dict(SMALL["qwen3_hd128_g2"])
    t = synth.generate(cfg)
    dev()
    flat = qdec.Model(cfg, t, max_seqs=4, max_ctx=256)
    paged = qdec.Model(cfg, t, max_seqs=4, max_ctx=256)
    paged.kv_paged(64, 12)
    yield cfg, t, flat, paged
    flat.close()
    paged.close()


def test_continuous_batching_matches_the_oracle(qwen3_pair):
    cfg, t, flat, _ = qwen3_pair
    om = OracleModel(cfg, t, max_ctx=256, n_seqs=4)
    run_schedule(flat, cfg, om)


def test_paged_cache_is_bit_identical_to_the_contiguous_one(qwen3_pair):
    cfg, t, flat, paged = qwen3_pair
    assert paged.kv_pages() == (64, 12, 12)
    a = run_schedule(flat, cfg)
    b = run_schedule(paged, cfg, pages=True)
    assert a.keys() == b.keys()
    for k in a:
        # decode attention adds its chunks' partials with f32 atomics, whose
        # order varies from run to run: agreement to f32 rounding, not bits
        assert rel_err(b[k], a[k]) < 1e-5, k
    om = OracleModel(cfg, t, max_ctx=256, n_seqs=4)
    run_schedule(paged, cfg, om, pages=True)


def test_paged_eight_heads_per_kv_head_matches_the_oracle():
    """Eight query heads per KV head run decode attention as two workgroups of
    four per KV head, which both place the KV head's rows (one of them appends
    the new key and value): the batching schedule on a paged cache, every
    logits row against the oracle."""
    cfg = dict(SMALL["gqa8_hd128"])
    t = synth.generate(cfg)
    m = qdec.Model(cfg, t, max_seqs=4, max_ctx=256)
    try:
        m.kv_paged(64, 12)
        om = OracleModel(cfg, t, max_ctx=256, n_seqs=4)
        run_schedule(m, cfg, om, pages=True)
    finally:
        m.close()


def test_paged_window_model_matches_the_oracle():
    """head_dim 256 (decode chunk 32), window 8, pages of 32: prefill tiles of
    16 keys on window layers start anywhere and straddle pages."""
    cfg = dict(SMALL["gemma_hd256_g4"])
    t = synth.generate(cfg)
    dev()
    with qdec.Model(cfg, t, max_seqs=2, max_ctx=200) as m:
        m.kv_paged(32, 9)
        om = OracleModel(cfg, t, max_ctx=200, n_seqs=2)
        V = cfg["vocab"]
        for s, T in ((1, 75), (0, 41)):
            prompt = synth.prompt(cfg, T, tag=f"w{s}")
            pl = torch.empty((T, V), dtype=torch.float32, device=dev())
            m.prefill(s, prompt, pl, None, all_logits=True)
            torch.cuda.synchronize()
            o = om.forward(s, prompt, all_logits=True)
            g = as_np(pl)
            for i in range(T):
                check_row(g[i], o[i])
        dl = torch.empty((2, V), dtype=torch.float32, device=dev())
        out = torch.empty(2, dtype=torch.int32, device=dev())
        cur = {0: 3, 1: 7}
        for step in range(10):
            m.decode_batch([1, 0], [cur[1], cur[0]], dl, out)
            torch.cuda.synchronize()
            g, got = as_np(dl), as_np(out).tolist()
            for r, s in enumerate((1, 0)):
                o = om.forward(s, [cur[s]])[0]
                check_row(g[r], o)
                cur[s] = got[r]


# One-layer models wide enough (QKV 3,072 rows, 2,112 gate/up pairs, 2,048
# down outputs, a 2,500-row head) for the matrix-core decode of 9..16 rows.
WIDE = dict(SMALL["qwen2_bias_hd64_g2"], n_layer=1, hidden=2048, n_head=16, n_head_kv=4, head_dim=128,
            ffn=2112, vocab=2500, embd_type="f32", tied=False)
WIDE_CASES = {
    "wide_q8_0_bias_silu": dict(WIDE, name="wide_q8_0_bias_silu", wtype="q8_0", seed=21),
    "wide_q4_0_gelu": dict(WIDE, name="wide_q4_0_gelu", wtype="q4_0", qkv_bias=False, act="gelu_tanh", seed=22),
    # a Q4_K_M-like mix (Q4_K, Q6_K for attn_v, ffn_down and the head); FFN
    # width a multiple of the 256-value super-block
    "wide_q4km": dict(WIDE, name="wide_q4km", wtype="q4_k", qkv_bias=False, ffn=2304, seed=23,
                      types={"attn_v": "q6_k", "ffn_down": "q6_k", "output": "q6_k"}),
}


@pytest.mark.parametrize("key,n", [("wide_q8_0_bias_silu", 12), ("wide_q4_0_gelu", 16), ("wide_q8_0_bias_silu", 9),
                                   ("wide_q4_0_gelu", 5), ("wide_q4km", 11)])
def test_decode_batch_of_five_to_sixteen_matches_the_oracle(key, n):
    """Five to sixteen decode rows run the QKV (RMSNorm prologue, bias),
    gate/up (pair epilogue, SiLU or gelu_tanh), down (residual add) and head
    projections on the matrix cores (Q8_0, Q4_0 and a Q4_K / Q6_K mix): every logits row
    of a few greedy steps over a shuffled slot order against the oracle, slots
    at different lengths."""
    cfg = dict(WIDE_CASES[key])
    t = synth.generate(cfg)
    dev()
    V = cfg["vocab"]
    with qdec.Model(cfg, t, max_seqs=n, max_ctx=96) as m:
        om = OracleModel(cfg, t, max_ctx=96, n_seqs=n)
        pl = torch.empty((1, V), dtype=torch.float32, device=dev())
        tok = torch.empty(1, dtype=torch.int32, device=dev())
        cur = {}
        for s in range(n):
            prompt = synth.prompt(cfg, 3 + 5 * s % 37, tag=f"b{s}")
            m.prefill(s, prompt, pl, tok)
            torch.cuda.synchronize()
            cur[s] = int(as_np(tok)[0])
            om.forward(s, prompt)
        rng = np.random.default_rng(n)
        dl = torch.empty((n, V), dtype=torch.float32, device=dev())
        out = torch.empty(n, dtype=torch.int32, device=dev())
        for step in range(4):
            seqs = [int(x) for x in rng.permutation(n)]
            m.decode_batch(seqs, [cur[s] for s in seqs], dl, out)
            torch.cuda.synchronize()
            g, got = as_np(dl), as_np(out).tolist()
            for r, s in enumerate(seqs):
                o = om.forward(s, [cur[s]])[0]
                check_row(g[r], o)
                assert token_agrees(got[r], o), (step, s)
                cur[s] = got[r]


def test_sampled_slot_uses_its_own_stream(qwen3_pair):
    cfg, t, flat, _ = qwen3_pair
    V = cfg["vocab"]
    flat.kv_reset()
    tok = torch.empty(1, dtype=torch.int32, device=dev())
    pl = torch.empty((1, V), dtype=torch.float32, device=dev())
    for s, T in ((1, 12), (3, 20)):
        flat.prefill(s, synth.prompt(cfg, T, tag=f"s{s}"), pl, tok)
    dl = torch.empty((2, V), dtype=torch.float32, device=dev())
    out = torch.empty(2, dtype=torch.int32, device=dev())
    cur = [5, 9]
    checked = 0
    for step in range(12):
        flat.decode_batch([3, 1], cur, dl, out, temperature=1.0, seed=33, step=step)
        torch.cuda.synchronize()
        g, got = as_np(dl), as_np(out).tolist()
        for r, s in enumerate((3, 1)):
            sc = sampler.scores(g[r], 1.0, 33, step, s)
            top2 = np.partition(sc, -2)[-2:]
            if top2[1] - top2[0] > 1e-4:
                assert got[r] == int(np.argmax(sc)), (step, s)
                checked += 1
        cur = got
    assert checked >= 16


def test_refusals_leave_the_handle_usable(qwen3_pair):
    cfg, t, flat, paged = qwen3_pair
    V = cfg["vocab"]
    pl = torch.empty((1, V), dtype=torch.float32, device=dev())
    dl = torch.empty((2, V), dtype=torch.float32, device=dev())
    out = torch.empty(2, dtype=torch.int32, device=dev())
    flat.kv_reset()
    flat.prefill(0, [1, 2, 3], pl)
    with pytest.raises(qdec.QdecError, match="in use"):
        flat.kv_paged(64, 4)
    with pytest.raises(qdec.QdecError, match="twice"):
        flat.decode_batch([0, 0], [1, 2], dl, out)
    with pytest.raises(qdec.QdecError, match="outside"):
        flat.decode_batch([4], [1], dl[:1], out[:1])
    flat.decode_batch([0], [4], dl[:1], out[:1])
    flat.kv_reset()
    with pytest.raises(qdec.QdecError, match="power of two"):
        flat.kv_paged(48, 4)
    with pytest.raises(qdec.QdecError, match="below the decode chunk"):
        flat.kv_paged(32, 4)
    # a pool of three pages: 150 positions take all of them
    cfg2 = dict(cfg)
    with qdec.Model(cfg2, t, max_seqs=2, max_ctx=256) as m:
        m.kv_paged(64, 3)
        m.prefill(0, synth.prompt(cfg, 150, tag="big"), pl)
        assert m.kv_pages() == (64, 3, 0)
        with pytest.raises(qdec.QdecError, match="exhausted"):
            m.prefill(1, [1, 2], pl)
        # the last page of sequence 0 has room: decode still works
        m.decode_batch([0], [7], dl[:1], out[:1])
        m.kv_truncate(0, 100)  # gives back one page
        assert m.kv_pages() == (64, 3, 1)
        m.prefill(1, [1, 2], pl)
        m.kv_reset()
        assert m.kv_pages() == (64, 3, 3)
        torch.cuda.synchronize()


def test_decode_chunk_that_is_not_a_power_of_two():
    """head_dim 256 with max_ctx 2,100: 32-position chunks would exceed the
    merge's 64 chunks, so the contiguous cache splits decode attention into
    48-position chunks (the prompt crosses two chunk boundaries); a paged cache
    of 64-position pages on the same model uses 64-position chunks.  Both match
    the oracle."""
    cfg = dict(SMALL["gemma_hd256_g4"])
    t = synth.generate(cfg)
    dev()
    V = cfg["vocab"]
    prompt = synth.prompt(cfg, 100, tag="np2")
    for paged in (False, True):
        with qdec.Model(cfg, t, max_seqs=1, max_ctx=2100) as m:
            if paged:
                m.kv_paged(64, 40)
            # the split the library chose: 48-position chunks (44 of them), or
            # the 64-position pages' chunk (33 of them)
            assert m.decode_chunks() == ((64, 33) if paged else (48, 44))
            om = OracleModel(cfg, t, max_ctx=120, n_seqs=1)
            pl = torch.empty((1, V), dtype=torch.float32, device=dev())
            tok = torch.empty(1, dtype=torch.int32, device=dev())
            m.prefill(0, prompt, pl, tok)
            torch.cuda.synchronize()
            check_row(as_np(pl)[0], om.forward(0, prompt)[0])
            dl = torch.empty((1, V), dtype=torch.float32, device=dev())
            out = torch.empty(1, dtype=torch.int32, device=dev())
            cur = int(as_np(tok)[0])
            for step in range(6):
                m.decode_batch([0], [cur], dl, out)
                torch.cuda.synchronize()
                o = om.forward(0, [cur])[0]
                check_row(as_np(dl)[0], o)
                cur = int(as_np(out)[0])
