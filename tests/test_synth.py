"""The seeded input generator: determinism, sizes and the encoder's error bound."""
import numpy as np

import synth
from oracle import blocks


def test_tensor_sizes_follow_block_layout():
    cfg = synth.get("c1")
    t = synth.generate(cfg, threads=2)
    down = t["blk.0.ffn_down.weight"]
    assert (down.rows, down.cols) == (256, 688)
    assert down.nbytes == 256 * 22 * 34          # 688 -> 22 blocks (padded to 704)
    assert t["token_embd.weight"].type == synth.T_F32 and t["token_embd.weight"].nbytes == 1024 * 256 * 4
    assert "output.weight" not in t
    for name, tt in t.items():
        assert tt.nbytes == synth.tensor_nbytes(tt.type, tt.rows, tt.cols), name


def test_generation_is_deterministic_and_thread_independent():
    cfg = dict(synth.get("c1"), n_layer=1)
    a = synth.generate(cfg, threads=1)
    b = synth.generate(cfg, threads=4)
    assert synth.manifest(a) == synth.manifest(b)
    assert np.array_equal(synth.prompt(cfg), synth.prompt(cfg))
    c = synth.generate(dict(cfg, seed=99), threads=1)
    assert synth.manifest(a)["blk.0.attn_q.weight"] != synth.manifest(c)["blk.0.attn_q.weight"]


def test_encoder_round_trip_bound():
    x = np.random.default_rng(0).standard_normal((64, 200)).astype(np.float32) * 0.02
    for tt, qmax in [(synth.T_Q8_0, 127), (synth.T_Q4_0, 7)]:
        raw = synth.encode(tt, x)
        back = blocks.dequant(tt, raw, 64, 200)
        nb = (200 + 31) // 32
        xp = np.concatenate([x, np.zeros((64, nb * 32 - 200), np.float32)], axis=1).reshape(64, nb, 32)
        amax = np.abs(xp).max(axis=2)
        d = (amax / (127.0 if tt == synth.T_Q8_0 else 8.0)).astype(np.float16).astype(np.float64)
        err = np.abs(back.astype(np.float64) - x).reshape(64, -1)
        errp = np.concatenate([err, np.zeros((64, nb * 32 - 200))], axis=1).reshape(64, nb, 32)
        # half a step; an element clipped at the positive end (Q4_0: +8 -> +7) is off
        # by up to one step, plus the fp16 rounding of d (amax/d <= 8 * (1 + 2^-11))
        bound = d[..., None] * (0.5 + 1e-6)
        clipped = (xp / np.where(d == 0, 1, d)[..., None]) > qmax + 0.5
        assert (errp <= np.where(clipped, d[..., None] * (1.0 + 2.0 ** -7), bound)).all()


def test_prompt_range_and_weight_stats():
    cfg = synth.get("c2")
    p = synth.prompt(cfg)
    assert p.dtype == np.int32 and p.shape == (512,) and p.min() >= 0 and p.max() < 151936
    cfg1 = synth.get("c1")
    t = synth.generate(cfg1, threads=2)
    w = blocks.dequant(synth.T_Q8_0, t["blk.1.attn_q.weight"].data, 256, 256)
    assert abs(w.std() - 0.02) < 0.001
