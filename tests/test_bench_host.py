"""Host-side checks of bench.py (no GPU): the refusal of several GPUs, the
algorithmic byte and flop counts behind the reported fractions, worked out
here by hand from the shapes and the GGUF block sizes, and the roofline
object's arithmetic and its guard on stale counter readings."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

# GGUF block sizes: bytes per 32 weights
Q4_0, Q8_0 = 18, 34


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_decode_step_bytes_of_the_8b_shape():
    """Llama-8B shape, Q4_0 everywhere, one sequence, KV length 1,100 before the
    step: the seven layer matrices, the untied head, the cache rows read and the
    new one written, one embedding row and the logits row."""
    cfg = dict(synth.CONFIGS["c3"])
    H, F, V, L = 4096, 14336, 128256, 32
    q, kv = 32 * 128, 8 * 128
    layer_weights = H * (q + 2 * kv) + q * H + 3 * H * F
    assert layer_weights == 218_103_808
    layer_bytes = layer_weights // 32 * Q4_0
    head = V * H // 32 * Q4_0
    pos = 1100
    cache = L * kv * 4 * 2 * (pos + 2)  # K and V rows in f32: pos + 1 keys read, one written
    embd_row = H // 32 * Q4_0
    want = L * layer_bytes + head + cache + embd_row + V * 4
    assert want == 4_510_768_384
    assert bench.step_bytes_decode(cfg, pos) == want


def test_decode_step_bytes_scale_with_the_batch_and_the_window():
    """Sixteen sequences share the weights but each reads its own cache rows,
    embedding row and logits row; a windowed layer reads at most `window` keys."""
    cfg = dict(synth.CONFIGS["c1"])
    one = bench.step_bytes_decode(dict(cfg, batch=1), 40)
    sixteen = bench.step_bytes_decode(dict(cfg, batch=16), 40)
    per_seq = (sixteen - one) / 15
    kv = cfg["n_head_kv"] * cfg["head_dim"]
    embd_row = cfg["hidden"] * 4  # f32 table
    assert per_seq == cfg["n_layer"] * kv * 8 * 42 + embd_row + cfg["vocab"] * 4
    windowed = dict(cfg, batch=1, window=8, window_period=2)  # layer 0 windowed, layer 1 global
    saved = one - bench.step_bytes_decode(windowed, 40)
    assert saved == kv * 8 * (41 - 8)


def test_prefill_flops_by_hand():
    """Two flops per multiply-add: the projections of T tokens, causal
    attention (scores and values: 4 hd flops per query-key pair per head) and
    the head on the last row."""
    cfg = dict(synth.CONFIGS["c1"])
    T = 5
    H, F, V, hd, nq, nkv = 256, 688, 1024, 64, 4, 2
    lin = 2 * T * (H * (nq + 2 * nkv) * hd + nq * hd * H + 3 * H * F)
    pairs = 1 + 2 + 3 + 4 + 5
    attn = 4 * hd * nq * pairs
    assert bench.prefill_flops(cfg, T) == 2 * (lin + attn) + 2 * V * H
    assert bench.prefill_attn_flops(cfg, T) == 2 * attn


def test_roofline_takes_the_class_with_the_most_time():
    kst = {
        "gemv_q4_0": dict(launches=100, ms=1.0, bytes=100 * 32e6, flops=0.0),
        "attn_decode": dict(launches=50, ms=0.4, bytes=50 * 9e6, flops=1.0),
        "gemm_q4_0": dict(launches=4, ms=0.9, bytes=1e9, flops=4 * 2e12),
    }
    r = bench.roofline_entry(kst)
    assert r["kernel"] == "gemv_q4_0" and r["bound"] == "hbm"
    assert r["achieved"] == pytest.approx(3.2e9 / 1e-3 / 1e9, rel=1e-9)  # 3,200 GB/s
    assert r["frac"] == pytest.approx(0.4, abs=1e-4)
    assert r["avg_launch_us"] == 10.0 and r["bytes_per_launch"] == 32_000_000
    kst["gemm_q4_0"]["ms"] = 2.0
    r = bench.roofline_entry(kst)
    assert r["kernel"] == "gemm_q4_0" and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(8e12 / 2e-3 / 1e12, rel=1e-3)  # 4,000 TFLOP/s of made-up work
    assert r["traffic"] is None


def test_stored_traffic_is_used_only_for_the_same_kernels(tmp_path, monkeypatch):
    """profiles/traffic_<config>.txt counts only while the kernel sources hash
    it names is the current one, and only for the kernel class it names."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "decoder_gguf_quantized_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// one kernel\n")
    h = bench.kernel_sources_hash()
    (tmp_path / "profiles" / "traffic_cx.txt").write_text(
        f"# note\nworkload: cx\nkernel: gemv_q4_0\nsources: {h}\nfetch_bytes: 1000\nwrite_bytes: 24\n")
    assert bench.measured_traffic("cx", "gemv_q4_0") == 1024
    assert bench.measured_traffic("cx", "gemv_q8_0") is None
    assert bench.measured_traffic("cy", "gemv_q4_0") is None
    (csrc / "k.hip").write_text("// one kernel, changed\n")
    assert bench.kernel_sources_hash() != h
    assert bench.measured_traffic("cx", "gemv_q4_0") is None
