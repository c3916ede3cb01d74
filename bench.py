"""Throughput of the quantized decoder forward pass on one MI355X.

One step = kv_reset, prefill of the prompt, then the decode steps (greedy, the
token chained on the device), all on seeded synthetic weights of the workload's
shape.  Prints one JSON line:
  value        decode tokens/s (whole job, one GPU)
  prefill_*    prefill tokens/s and FP32-MFMA utilisation
  hbm_frac     decode algorithmic bytes per step / decode time / 8 TB/s
  roofline     the dominant kernel's algorithmic bytes / its average launch time
               (HIP events on the launch stream, over a second pass of the timed steps)
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]
"""
import argparse
import json
import os
import sys
import time

if "--cpu-threads" in sys.argv:  # BLAS thread counts are fixed when numpy first loads
    _n = sys.argv[sys.argv.index("--cpu-threads") + 1]
    for _k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[_k] = _n

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
FP32_MFMA_PEAK = 157.3e12  # FLOP/s, MI355X dense FP32 matrix
BF16_MFMA_PEAK = 2.5e15    # FLOP/s, MI355X dense BF16 matrix
PREFILL_TERMS = {"f32": 0, "bf16x3": 3, "bf16": 1}
# mixed-type weight sets, as GGUF files ship them (the type of each matrix)
WEIGHT_MIXES = {
    "q4_k_m": dict(wtype="q4_k", embd_type="q4_k", types={"attn_v": "q6_k", "ffn_down": "q6_k", "output": "q6_k"}),
}


def step_bytes_decode(cfg, pos):
    """Algorithmic HBM bytes of one decode step at KV length ``pos`` (before the step)."""
    import synth
    B = cfg["batch"]
    specs = synth.tensor_specs(cfg)
    layer_w = sum(synth.tensor_nbytes(t, r, c) for n, t, r, c, k in specs if k == "matrix" and n.startswith("blk."))
    embd = [s for s in specs if s[0] == "token_embd.weight"][0]
    embd_bytes = synth.tensor_nbytes(embd[1], embd[2], embd[3])
    head = [s for s in specs if s[0] == "output.weight"]
    head_bytes = synth.tensor_nbytes(head[0][1], head[0][2], head[0][3]) if head else embd_bytes
    row = embd_bytes / embd[2]
    kv = 0
    for l in range(cfg["n_layer"]):
        n_keys = pos + 1
        if not synth.layer_is_global(cfg, l):
            n_keys = min(n_keys, cfg["window"])
        kv += cfg["n_head_kv"] * cfg["head_dim"] * 8 * (n_keys + 1)  # read keys + write the new one
    return layer_w + head_bytes + B * (kv + row + cfg["vocab"] * 4)


def prefill_attn_flops(cfg, T):
    import synth
    hd, nq = cfg["head_dim"], cfg["n_head"]
    attn = 0
    for l in range(cfg["n_layer"]):
        w = 0 if synth.layer_is_global(cfg, l) else cfg["window"]
        attn += 4 * hd * nq * sum(min(i + 1, w) if w else i + 1 for i in range(T))
    return attn


def prefill_flops(cfg, T):
    H, hd, nq, nkv, F, V = (cfg[k] for k in ("hidden", "head_dim", "n_head", "n_head_kv", "ffn", "vocab"))
    lin = 2 * T * (H * (nq + 2 * nkv) * hd + nq * hd * H + 3 * H * F)
    attn = 0
    for l in range(cfg["n_layer"]):
        import synth
        w = 0 if synth.layer_is_global(cfg, l) else cfg["window"]
        keys = sum(min(i + 1, w) if w else i + 1 for i in range(T))
        attn += 4 * hd * nq * keys
    return cfg["n_layer"] * lin + attn + 2 * V * H


def cpu_baseline(cfg, tensors, budget_s=20.0):
    """The oracle as it stands, timed on the host: a short prefill, then decode
    steps until the budget is spent.  Returns decode tokens/s and the sample.

    Models whose float64 weights would not fit a few GB of host memory (the
    8B shape: 60 GB) run the oracle on their first ``nl`` layers (the same
    tensors, the full LM head), and the per-token time is extrapolated as
    n_layer / nl times the blocks' time plus the head's time, which is timed on
    its own; the sample string says so."""
    from oracle import OracleModel
    import synth
    cores = len(os.sched_getaffinity(0))
    T0 = min(32, cfg["prompt_len"])
    prompt = synth.prompt(cfg, T0)
    n_layer = cfg["n_layer"]
    layer_weights = sum(r * c for n, _t, r, c, k in synth.tensor_specs(cfg) if k == "matrix" and n.startswith("blk."))
    nl = n_layer if layer_weights * 8 <= 6e9 else max(1, int(6e9 // (layer_weights * 8 / n_layer)))
    nl = min(nl, n_layer)
    scfg = dict(cfg, n_layer=nl)
    om = OracleModel(scfg, tensors, max_ctx=T0 + 64)
    om.mat(om.lm_head_name())  # decoded once, before any timed work
    t0 = time.perf_counter()
    logits = om.forward(0, prompt)
    t_pre = time.perf_counter() - t0
    tok = int(np.argmax(logits[-1]))
    n, t_dec, t_head = 0, 0.0, 0.0
    while n < 48 and (t_dec < budget_s or n < 2):
        t0 = time.perf_counter()
        x = om.hidden(0, [tok])
        t1 = time.perf_counter()
        logits = om.head(x[-1:])
        t2 = time.perf_counter()
        t_dec += t2 - t0
        t_head += t2 - t1
        tok = int(np.argmax(logits[-1]))
        n += 1
    per_tok = ((t_dec - t_head) * n_layer / nl + t_head) / n
    what = "" if nl == n_layer else (f" on the first {nl} of {n_layer} layers (float64 weights of all layers would "
                                     f"need {layer_weights * 8 / 1e9:.0f} GB), per-token time extrapolated as "
                                     f"{n_layer}/{nl} x blocks + head")
    return dict(value=1.0 / per_tok, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{cfg['name']}: {T0}-token prefill ({t_pre:.1f} s), then {n} greedy decode steps timed "
                       f"({t_dec:.1f} s){what}; float64 numpy, {cores} host threads")


def cpu_oracle_full(cfg, threads):
    """The oracle over a whole workload (prefill of the full prompt, then every
    greedy decode step), timed with perf_counter; ``threads`` host threads.
    Returns one JSON-able record.  Runs without a GPU."""
    from oracle import OracleModel
    import synth
    tensors = synth.generate(cfg)
    T, N = cfg["prompt_len"], cfg["decode_steps"]
    om = OracleModel(cfg, tensors, max_ctx=T + N + 1)
    prompt = synth.prompt(cfg)
    t0 = time.perf_counter()
    logits = om.forward(0, prompt)
    t_pre = time.perf_counter() - t0
    print(f"[cpu-oracle-full] {cfg['name']}: prefill of {T} tokens {t_pre:.1f} s", file=sys.stderr, flush=True)
    tok = int(np.argmax(logits[-1]))
    t0 = time.perf_counter()
    for i in range(N):
        logits = om.forward(0, [tok])
        tok = int(np.argmax(logits[-1]))
        if (i + 1) % 16 == 0:
            print(f"[cpu-oracle-full] {cfg['name']}: decode step {i + 1}/{N}, {time.perf_counter() - t0:.1f} s",
                  file=sys.stderr, flush=True)
    t_dec = time.perf_counter() - t0
    return dict(workload=cfg["name"], kind="oracle", cores=threads, prompt=T, decode_steps=N,
                prefill_s=round(t_pre, 3), prefill_tokens_per_s=round(T / t_pre, 3),
                decode_s=round(t_dec, 3), decode_tokens_per_s=round(N / t_dec, 3),
                note="float64 numpy; prefill includes decoding every matrix once to float64")


def kernel_sources_hash():
    """sha256 (first 16 hex) of the device sources (csrc/*.hip and *.hpp in
    name order: the kernels and their launches; the host-only model-file
    reader is left out), to tell whether stored counter readings still
    describe the kernels being timed."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "decoder_gguf_quantized_amd", "csrc", "*"))):
        if f.endswith((".hip", ".hpp")):
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(config, kernel):
    """HBM bytes per dispatch of ``kernel`` from the committed rocprofv3 --pmc
    summary (profiles/traffic_<config>.txt), or None when there is none or the
    kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel") != kernel or kv.get("sources") != kernel_sources_hash():
        return None
    return round(float(kv["fetch_bytes"]) + float(kv["write_bytes"]))


def roofline_entry(kst, config=None):
    """Roofline object for the kernel class with the most measured time."""
    dname, d = max(kst.items(), key=lambda kv: kv[1]["ms"])
    if d["flops"] and d["bytes"] and dname.startswith("gemm"):
        achieved = d["flops"] / (d["ms"] / 1e3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=157.3, unit="TFLOP/s",
                    frac=round(achieved / 157.3, 4), traffic=None)
    else:
        achieved = d["bytes"] / (d["ms"] / 1e3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=8000.0, unit="GB/s",
                    frac=round(achieved / 8000.0, 4), traffic=None)
    roof.update(kernel=dname, launches=d["launches"], avg_launch_us=round(d["ms"] * 1e3 / d["launches"], 2),
                bytes_per_launch=round(d["bytes"] / d["launches"]))
    if config:
        roof["traffic"] = measured_traffic(config, dname)
    return roof


def bench_batched(cfg, args):
    """Batched long-context decode: B sequences over preset K/V caches of P
    positions, N steps of temperature sampling.  One step = the N decode steps
    (each sequence rolled back to P first)."""
    import torch

    import decoder_gguf_quantized_amd as qdec
    import synth
    dev = torch.device("cuda:0")
    if args.decode_steps is not None:
        cfg["decode_steps"] = args.decode_steps
    if args.batch is not None:  # another number of sequences (the workload's name says it)
        import re
        cfg["batch"] = args.batch
        cfg["name"] = re.sub(r"-b\d+", f"-b{args.batch}", cfg["name"])
    B, P, N, V = cfg["batch"], cfg["preset_kv"], cfg["decode_steps"], cfg["vocab"]
    tensors = synth.generate(cfg)
    model = qdec.Model(cfg, tensors, max_seqs=B, max_ctx=P + N + 1)
    if args.kv_page:  # a pool that holds every sequence at its final length
        per_seq = -(-(P + N + 1) // args.kv_page)
        model.kv_paged(args.kv_page, B * per_seq)
    for s, l, k, v in synth.preset_kv_all(cfg):
        model.kv_write(s, l, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev))
    torch.cuda.synchronize()
    first = synth.first_tokens(cfg)
    dl = torch.empty((B, V), dtype=torch.float32, device=dev)
    toks = torch.empty((N + 1, B), dtype=torch.int32, device=dev)
    toks[0].copy_(torch.from_numpy(first))
    stream = torch.cuda.current_stream()
    seed, temp = cfg["seed"], cfg["temperature"]
    top_p = 1.0 if args.top_p is None else args.top_p

    def one_step():
        for s in range(B):
            model.kv_truncate(s, P)
        for i in range(N):
            model.decode_step(toks[i], dl, toks[i + 1], temperature=temp, seed=seed, step=i, top_p=top_p)

    def run(k):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(k):
            one_step()
        e1.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1)

    for _ in range(args.warmup):
        run(1)
    wall, ms = run(args.steps)
    model.kernel_timing(True)
    run(args.steps)
    kst = model.kernel_timing(False)
    model.close()
    tok_s = args.steps * B * N / (ms / 1e3)
    bytes_dec = sum(step_bytes_decode(cfg, P + i) for i in range(N)) * args.steps
    line = {
        "metric": "decode tokens/sec + HBM GB/s fraction; prefill tokens/sec + MFMA util",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: {B} sequences x {P} preset KV positions, {N} decode steps, "
                               f"temperature {temp} (Gumbel-max over Philox4x64-10)"
                               + (f", top-p {top_p}" if top_p < 1 else ""),
                   "batch": B, "preset_kv": P, "decode_steps": N, "weights": cfg["wtype"],
                   "kv_page": args.kv_page or None},
        "decode_hbm_frac": round(bytes_dec / (ms / 1e3) / HBM_PEAK, 4),
        "roofline": roofline_entry(kst, cfg.get("key")),
        "kernels": {k: dict(launches=v["launches"], ms=round(v["ms"], 3)) for k, v in sorted(kst.items())},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_batched(cfg, tensors)
    print(json.dumps(line), flush=True)


def cpu_baseline_batched(cfg, tensors, budget_s=20.0):
    """The oracle on sequence 0 of the batched workload: its preset cache, then
    sampled decode steps until the budget is spent."""
    from oracle import OracleModel, sampler
    import synth
    cores = len(os.sched_getaffinity(0))
    P = cfg["preset_kv"]
    om = OracleModel(cfg, tensors, max_ctx=P + 16)
    for s, l, k, v in synth.preset_kv_all(cfg, seqs=[0]):
        om.kv_write(0, l, k, v)
    om.set_kv_len(0, P)
    tok = int(synth.first_tokens(cfg)[0])
    n, t = 0, 0.0
    while n < 8 and (t < budget_s or n < 2):
        t0 = time.perf_counter()
        lg = om.forward(0, [tok])[0]
        tok = sampler.sample(lg, cfg["temperature"], cfg["seed"], n, 0)
        t += time.perf_counter() - t0
        n += 1
    return dict(value=n / t, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{cfg['name']}: sequence 0 of {cfg['batch']}, {P} preset KV positions, {n} sampled decode "
                       f"steps timed ({t:.1f} s), float64 numpy, {cores} host threads")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c3",
                    help="workload: c3 (default: the 8B shape, Q4_0), c1, c2, c4, c5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-page", type=int, default=0,
                    help="paged KV cache with pages of this many positions (0: contiguous cache)")
    ap.add_argument("--weights", default=None, choices=sorted(WEIGHT_MIXES),
                    help="re-type the workload's matrices, e.g. q4_k_m: Q4_K with Q6_K attn_v, ffn_down and head")
    ap.add_argument("--decode-steps", type=int, default=None, help="override the workload's decode steps (profiling runs)")
    ap.add_argument("--batch", type=int, default=None,
                    help="batched workload only: number of sequences (default: the workload's 16)")
    ap.add_argument("--prefill-precision", default="f32", choices=sorted(PREFILL_TERMS),
                    help="operand precision of the prefill projections (default f32)")
    ap.add_argument("--top-p", type=float, default=None,
                    help="batched workload only: restrict sampling to the top-p nucleus (default: none)")
    ap.add_argument("--cpu-oracle-full", default=None, metavar="CONFIG",
                    help="time the CPU oracle over the whole workload (no GPU) and print its record")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="with --cpu-oracle-full: host threads (default: all available)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device-to-device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    cores = len(os.sched_getaffinity(0))
    if args.cpu_oracle_full:
        n = args.cpu_threads or cores  # (set in the environment at import when given)
        import synth
        print(json.dumps(cpu_oracle_full(synth.get(args.cpu_oracle_full), n)), flush=True)
        return
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    os.environ.setdefault("OPENBLAS_NUM_THREADS", str(cores))
    import torch

    import decoder_gguf_quantized_amd as qdec
    import synth

    cfg = synth.get(args.config)
    cfg["key"] = args.config
    if args.weights:
        cfg.update(WEIGHT_MIXES[args.weights])
        cfg["key"] = f"{args.config}-{args.weights}"
    if args.copy_calibration:
        a = torch.empty(64 << 20, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if cfg["preset_kv"]:
        return bench_batched(cfg, args)
    tensors = synth.generate(cfg)
    dev = torch.device("cuda:0")
    if args.decode_steps is not None:
        cfg["decode_steps"] = args.decode_steps
    T, N, V = cfg["prompt_len"], cfg["decode_steps"], cfg["vocab"]
    prompt = synth.prompt(cfg)
    model = qdec.Model(cfg, tensors, max_seqs=1, max_ctx=T + N + 1)
    if args.kv_page:
        model.kv_paged(args.kv_page, -(-(T + N + 1) // args.kv_page))
    model.set_prefill_precision(args.prefill_precision)
    pl = torch.empty(V, dtype=torch.float32, device=dev)
    dl = torch.empty((N, V), dtype=torch.float32, device=dev)
    toks = torch.empty((N + 1, 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def one_step(ev):
        model.kv_reset()
        ev[0].record(stream)
        model.prefill(0, prompt, pl, toks[0])
        ev[1].record(stream)
        for s in range(N):
            model.decode_step(toks[s], dl[s:s + 1], toks[s + 1])
        ev[2].record(stream)

    def run(k):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(k)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(k):
            one_step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        pre = [e[0].elapsed_time(e[1]) for e in evs]
        dec = [e[1].elapsed_time(e[2]) for e in evs]
        return wall, pre, dec

    for _ in range(args.warmup):
        run(1)
    wall, pre_ms, dec_ms = run(args.steps)
    # the exact three-term bf16 prefill alongside the default f32 one (same prompt)
    alt_pre_ms = None
    if args.prefill_precision == "f32":
        model.set_prefill_precision("bf16x3")
        run(1)
        alt_pre_ms = [run(1)[1][0] for _ in range(args.steps)]
        model.set_prefill_precision("f32")
    # second pass of the same steps with per-dispatch events for the roofline figure
    model.kernel_timing(True)
    run(args.steps)
    kst = model.kernel_timing(False)
    model.close()

    dec_tok_s = args.steps * N / (sum(dec_ms) / 1e3)
    pre_tok_s = args.steps * T / (sum(pre_ms) / 1e3)
    bytes_dec = sum(step_bytes_decode(cfg, T + s) for s in range(N))
    hbm_frac = bytes_dec / (np.mean(dec_ms) / 1e3) / HBM_PEAK
    # f32 path: algorithmic flops against the FP32 matrix peak.  bf16 paths:
    # also the bf16 MFMA work actually issued (terms x the projections' flops)
    # against the BF16 matrix peak.
    pre_s = np.mean(pre_ms) / 1e3
    mfma_util = prefill_flops(cfg, T) / pre_s / FP32_MFMA_PEAK
    nt = PREFILL_TERMS[args.prefill_precision]
    line = {
        "metric": "decode tokens/sec + HBM GB/s fraction; prefill tokens/sec + MFMA util",
        "value": round(dec_tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}, {(args.weights or cfg['wtype']).upper()} weights, prompt {T}, "
                               f"decode {N} greedy, batch 1",
                   "prompt": T, "decode_steps": N, "batch": 1, "weights": args.weights or cfg["wtype"],
                   "kv_page": args.kv_page or None},
        "prefill_tokens_per_s": round(pre_tok_s, 1),
        "prefill_mfma_util": round(float(mfma_util), 4),
        "prefill_precision": args.prefill_precision,
        "decode_hbm_frac": round(float(hbm_frac), 4),
        "decode_ms_per_token": round(float(np.mean(dec_ms)) / N, 4),
        "roofline": roofline_entry(kst, cfg["key"]),
        "kernels": {k: dict(launches=v["launches"], ms=round(v["ms"], 3)) for k, v in sorted(kst.items())},
    }
    if alt_pre_ms:
        line["prefill_tokens_per_s_bf16x3"] = round(args.steps * T / (sum(alt_pre_ms) / 1e3), 1)
    if nt:
        proj = prefill_flops(cfg, T) - prefill_attn_flops(cfg, T)
        line["prefill_bf16_mfma_util"] = round(float(nt * proj / pre_s / BF16_MFMA_PEAK), 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, tensors)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
