"""Host-only tests of the Python binding against a recording stand-in of
libqdec (tests/standin/qdec_standin.c), selected with QDEC_LIB: ownership
(freed exactly once, idempotent close, no copies or pickles), thread affinity,
integer and tensor checks made before any call reaches the library, and the
mapping of status codes to exceptions (tessl `python/README.md`, "Handle
ownership, closing and errors" and "Build and test").  No GPU is needed."""
import ctypes
import os
import re
import shutil
import subprocess
import threading

import numpy as np
import pytest

import decoder_gguf_quantized_amd as qdec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "standin", "qdec_standin.c")
HEADER = os.path.join(ROOT, "include", "qdec.h")

CFG = dict(n_layer=1, hidden=64, n_head=1, n_head_kv=1, head_dim=64, ffn=64, vocab=16, rms_eps=1e-6,
           rope_theta=1e4, rope_theta_local=1e4, window=0, window_period=0, qk_norm=0, sandwich_norm=0, act="silu")


class Rec:
    def __init__(self, name):
        self.name, self.type, self.rows, self.cols = name, 0, 1, 64
        self.data = np.zeros(256, dtype=np.uint8)


@pytest.fixture(scope="module")
def standin_path(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    out = str(tmp_path_factory.mktemp("standin") / "libqdec_standin.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC", "-o", out, SRC],
                   check=True)
    return out


@pytest.fixture
def S(standin_path, monkeypatch):
    """The binding loaded against the stand-in; yields the stand-in's CDLL."""
    monkeypatch.setenv("QDEC_LIB", standin_path)
    monkeypatch.setattr(qdec, "_lib", None)
    L = qdec.lib()
    assert os.path.samefile(L._name, standin_path)
    L.standin_log.restype = ctypes.c_char_p
    L.standin_reset()
    yield L
    L.standin_reset()


def log(S):
    return S.standin_log().decode().splitlines()


def model():
    return qdec.Model(CFG, [Rec("token_embd.weight")], max_seqs=2, max_ctx=32)


def test_standin_exports_every_declared_function(standin_path):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(qdec_[a-z_0-9]+)\s*\(", text)))
    L = ctypes.CDLL(standin_path)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, f"stand-in lacks {missing}"


def test_load_passes_the_null_stream_without_a_gpu(S):
    m = model()
    assert log(S)[0].startswith("load_weights n_tensors=1 max_seqs=2 max_ctx=32")
    if not __import__("torch").cuda.is_available():
        assert "stream=(nil)" in log(S)[0]
    m.close()


def test_freed_exactly_once(S):
    m = model()
    m.close()
    m.close()
    assert S.standin_frees() == 1 and S.standin_double_frees() == 0
    assert m.closed
    with pytest.raises(qdec.QdecError, match="closed"):
        m.kv_reset()
    with model() as m2:
        m2.kv_reset(0)
    assert S.standin_frees() == 2
    m3 = model()
    del m3  # the finaliser frees a handle its owner forgot
    assert S.standin_frees() == 3 and S.standin_double_frees() == 0


def test_copy_and_pickle_are_refused(S):
    import copy
    import pickle
    m = model()
    for f in (copy.copy, copy.deepcopy, pickle.dumps):
        with pytest.raises(TypeError):
            f(m)
    m.close()
    assert S.standin_frees() == 1


def test_thread_affinity(S):
    m = model()
    errs = []

    def use():
        try:
            m.kv_reset(0)
        except qdec.QdecError as e:
            errs.append(str(e))

    t = threading.Thread(target=use)
    t.start()
    t.join()
    assert errs and "thread" in errs[0]
    assert not any(x.startswith("kv_reset") for x in log(S))

    def close():
        try:
            m.close()
        except qdec.QdecError as e:
            errs.append(str(e))

    t = threading.Thread(target=close)
    t.start()
    t.join()
    assert "leaked" in errs[-1]
    assert S.standin_frees() == 0  # a handle is never freed from a foreign thread


def test_integers_are_range_checked_before_the_call(S):
    m = model()
    n0 = len(log(S))
    for call in (lambda: m.kv_truncate(2 ** 31, 0), lambda: m.kv_reset(-(2 ** 31) - 1), lambda: m.kv_len(True),
                 lambda: m.kv_paged(2 ** 40, 1), lambda: m.kv_truncate(0, 1.5)):
        with pytest.raises(qdec.QdecError):
            call()
    assert len(log(S)) == n0
    m.kv_truncate(1, 0)
    assert log(S)[-1] == "kv_truncate 1 0"
    m.close()


def test_tensors_are_checked_before_the_call(S):
    import torch
    m = model()
    n0 = len(log(S))
    with pytest.raises(qdec.QdecError, match="GPU|torch tensor"):
        m.prefill(0, [1, 2, 3], torch.zeros(16))  # host logits buffer
    with pytest.raises(qdec.QdecError, match="GPU|torch tensor"):
        m.decode_step([1], np.zeros(16, np.float32), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(qdec.QdecError, match="int32"):
        m.prefill(0, [2 ** 40], torch.zeros(16))
    with pytest.raises(qdec.QdecError, match="1-D"):
        m.prefill(0, [[1, 2]], torch.zeros(16))
    assert len(log(S)) == n0
    m.close()


def test_status_codes_map_to_exceptions(S):
    m = model()
    S.standin_force(1)
    with pytest.raises(qdec.QdecError) as e:
        m.kv_reset(0)
    assert type(e.value) is qdec.QdecError and "refused" in str(e.value)
    m.kv_reset(0)  # a refusal leaves the handle usable
    assert not m.poisoned
    S.standin_force(2)
    with pytest.raises(qdec.QdecPoisoned, match="internal"):
        m.kv_reset(0)
    # the binding frees a poisoned handle and refuses further use
    assert m.closed and S.standin_frees() == 1
    with pytest.raises(qdec.QdecError, match="closed"):
        m.kv_reset(0)
    m.close()
    assert S.standin_frees() == 1 and S.standin_double_frees() == 0


def test_injected_fault_poisons_through_the_binding(S):
    m = model()
    m.debug_inject_fault()
    assert log(S)[-1] == "debug_inject_fault 1"
    with pytest.raises(qdec.QdecPoisoned):
        m.set_prefill_precision("bf16x3")
    assert m.closed and S.standin_frees() == 1


def test_unknown_precision_is_refused_by_the_binding(S):
    m = model()
    n0 = len(log(S))
    with pytest.raises(qdec.QdecError, match="precision"):
        m.set_prefill_precision("fp8")
    assert len(log(S)) == n0
    m.close()
