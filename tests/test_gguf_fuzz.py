"""The library's GGUF reader and definition compiler on corrupted input,
host-only.

- gguf.cpp is built with AddressSanitizer and UndefinedBehaviorSanitizer (g++,
  no GPU code) into a small harness, which parses thousands of seeded
  mutations of valid files (byte flips, truncations, oversized counts and
  lengths, overwritten u64 fields) and of definition texts (lines dropped,
  repeated, swapped, cut; characters and words replaced).  Every one must be
  parsed or refused; a crash, out-of-bounds access or undefined behaviour
  fails the test.
- Soundness of the compiler: every mutated definition the library accepts
  must compute, when the oracle interprets it statement by statement, exactly
  what the oracle's fixed block computes with the shape the library derived.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import synth
import synth.gguf as sg

HERE = os.path.dirname(os.path.abspath(__file__))
ARCH_CASES = (("qwen2", "qwen2_bias_hd64_g2"), ("gemma3", "gemma_hd256_g4"), ("llama", "llama_q4_hd64_g4"),
              ("qwen3", "qwen3_hd128_g2"))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("fuzz") / "gguf_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "fuzz", "gguf_fuzz.cpp"),
           os.path.join(ROOT, "decoder_gguf_quantized_amd", "csrc", "gguf.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        if "cannot find" in r.stderr and "asan" in r.stderr:
            pytest.skip("no sanitizer runtime: " + r.stderr[-300:])
        raise RuntimeError(r.stderr)
    return out


def seeds(tmp_path):
    """Valid files to mutate: the hand-laid fixture and two written models."""
    txt = open(os.path.join(HERE, "golden", "tiny.gguf.hex")).read()
    out = [bytes(int(x, 16) for ln in txt.splitlines() for x in ln.split("#")[0].split())]
    from tests.gpu_helpers import SMALL
    for key in ("qwen2_bias_hd64_g2", "q4km_mixed_hd64_g4"):
        cfg = dict(SMALL[key])
        cfg.update(n_layer=1, vocab=64, hidden=256, ffn=256)
        p = sg.write(str(tmp_path / f"{key}.gguf"), cfg, synth.generate(cfg), vocab_strings=True)
        out.append(open(p, "rb").read())
    return out


BIG = [2 ** 63, 2 ** 64 - 1, 2 ** 32, 2 ** 40, 1 << 20]
ODD_TYPES = [9, 13, 100, 2 ** 31]


def mutate(b, rng):
    b = bytearray(b)
    kind = rng.integers(0, 6)
    if kind == 0:  # flip a few bytes in the header region
        for _ in range(rng.integers(1, 8)):
            i = int(rng.integers(0, min(len(b), 4096)))
            b[i] = int(rng.integers(0, 256))
    elif kind == 1:  # truncate
        b = b[:int(rng.integers(0, len(b)))]
    elif kind == 2:  # an oversized u64 (count / length / offset / dim) somewhere in the header
        i = int(rng.integers(0, max(1, min(len(b), 4096) - 8)))
        b[i:i + 8] = struct.pack("<Q", BIG[int(rng.integers(0, len(BIG)))])
    elif kind == 3:  # a small u64 count overwritten at the counts
        at = int(rng.choice([8, 16]))
        b[at:at + 8] = struct.pack("<Q", int(rng.integers(0, 1 << 16)))
    elif kind == 4:  # random bytes after a valid prefix
        i = int(rng.integers(0, len(b)))
        b[i:] = rng.integers(0, 256, size=len(b) - i, dtype=np.uint8).tobytes()
    else:  # a u32 type field set to an unknown or container type
        i = int(rng.integers(0, max(1, min(len(b), 4096) - 4)))
        b[i:i + 4] = struct.pack("<I", ODD_TYPES[int(rng.integers(0, len(ODD_TYPES)))])
    return bytes(b)


def test_corrupted_files_are_parsed_or_refused(harness, tmp_path):
    rng = np.random.default_rng(2024)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    parsed = 0
    for s, base in enumerate(seeds(tmp_path)):
        for b0 in range(0, 700, 350):
            paths = []
            for i in range(b0, b0 + 350):
                p = tmp_path / f"m{s}_{i}.gguf"
                p.write_bytes(mutate(base, rng))
                paths.append(p)
            r = subprocess.run([harness] + [str(p) for p in paths], capture_output=True, text=True, env=env,
                               timeout=600)
            assert r.returncode == 0, (s, b0, r.stdout[-500:], r.stderr[-3000:])
            assert r.stdout.startswith("ok ")
            parsed += int(r.stdout.split()[1])
            for p in paths:
                p.unlink()
    # mutations in the tensor data leave a valid file: the model shape is
    # reached, not only the early refusals
    assert parsed > 200


PUNCT = "(),=|{}.#09- \t\xff"


def mutate_text(t, rng):
    lines = t.split("\n")
    kind = rng.integers(0, 7)
    i = int(rng.integers(0, len(lines)))
    if kind == 0:  # drop a line
        del lines[i]
    elif kind == 1:  # repeat a line
        lines.insert(i, lines[int(rng.integers(0, len(lines)))])
    elif kind == 2:  # swap two lines
        j = int(rng.integers(0, len(lines)))
        lines[i], lines[j] = lines[j], lines[i]
    elif kind == 3:  # cut the text anywhere
        return t[:int(rng.integers(0, len(t)))]
    elif kind == 4:  # replace a character with punctuation, a digit or a byte above ASCII
        if lines[i]:
            k = int(rng.integers(0, len(lines[i])))
            c = PUNCT[int(rng.integers(0, len(PUNCT)))]
            lines[i] = lines[i][:k] + c + lines[i][k + 1:]
    elif kind == 5:  # swap two words across the text
        words = t.split()
        a, b = words[int(rng.integers(0, len(words)))], words[int(rng.integers(0, len(words)))]
        return t.replace(a, "\0TMP").replace(b, a).replace("\0TMP", b)
    else:  # very long names and numbers
        lines[i] = lines[i].replace("{i}", "{i}" * 50).replace("6", "9" * 40)
    return "\n".join(lines)


def test_corrupted_definitions_are_compiled_or_refused(harness, tmp_path):
    """Mutated definition texts against valid files of their architectures:
    every one compiles or is refused, and the unmutated text compiles."""
    rng = np.random.default_rng(77)
    args = []
    for arch, key in ARCH_CASES:
        cfg = small_cfg(arch, key)
        g = sg.write(str(tmp_path / f"{arch}.gguf"), cfg, synth.generate(cfg))
        text = sg.archdef_text(arch)
        for i in range(400):
            d = tmp_path / f"{arch}_{i}.archdef"
            d.write_bytes(mutate_text(text, rng).encode("utf-8"))
            args += ["-d", str(d), g]
        d = tmp_path / f"{arch}.archdef"
        d.write_text(text)
        args += ["-d", str(d), g]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([harness] + args, capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-500:], r.stderr[-3000:])
    ok = int(r.stdout.split()[1])
    assert ok >= 4, r.stdout


def small_cfg(arch, key):
    from tests.gpu_helpers import SMALL
    cfg = dict(SMALL[key])
    cfg.update(n_layer=1, vocab=64, hidden=256, ffn=256)
    if arch == "gemma3":
        cfg.update(n_layer=6, window_period=6)
    return cfg


@pytest.mark.parametrize("arch,key", ARCH_CASES)
def test_accepted_definitions_compute_what_the_library_runs(tmp_path, arch, key):
    """A definition the compiler accepts is run by the kernels as the fixed
    block with the derived shape (activation, biases, q/k norms, sandwich
    norms, rope bases, window pattern, head).  The oracle's statement-by-statement
    run of each accepted mutation must equal its fixed-block model of that
    shape, to rounding order (1e-12 of the largest logit)."""
    import decoder_gguf_quantized_amd as qdec
    from oracle import OracleModel, gguf
    from oracle import archdef as ad
    if not os.path.exists(qdec.lib_path()):
        from decoder_gguf_quantized_amd import build
        build.build()
    rng = np.random.default_rng(100 + [a for a, _ in ARCH_CASES].index(arch))
    cfg = small_cfg(arch, key)
    tens = synth.generate(cfg)
    path = sg.write(str(tmp_path / f"{arch}.gguf"), cfg, tens)
    G = gguf.read(path)
    text = sg.archdef_text(arch)
    prompt = [3, 5, 7, 11]
    accepted = 0
    for i in range(120):
        t = mutate_text(text, rng) if i else text
        try:
            shape = qdec.gguf_config(path, t)
        except qdec.QdecError:
            continue
        accepted += 1
        got = ad.Interpreter(ad.parse(t), G, max_ctx=8).forward(0, prompt, all_logits=True)
        want = OracleModel(shape, tens, max_ctx=8).forward(0, prompt, all_logits=True)
        err = float(np.max(np.abs(got - want)) / np.max(np.abs(want)))
        assert err < 1e-12, (i, err, t)
    assert accepted >= 20
