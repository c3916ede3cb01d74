"""Host-only checks of the C ABI: the library loads, exports every function
include/qdec.h declares, and refuses bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

import decoder_gguf_quantized_amd as qdec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qdec.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qdec.lib_path()):
        from decoder_gguf_quantized_amd import build
        build.build()
    return qdec.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qdec_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), f"{n} missing from libqdec.so"


def test_abi_version(L):
    want = int(re.search(r"#define QDEC_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.qdec_abi_version() == want


def cfg(**kw):
    c = dict(n_layer=1, hidden=64, n_head=1, n_head_kv=1, head_dim=64, ffn=64, vocab=16, rms_eps=1e-6,
             rope_theta=1e4, rope_theta_local=1e4, window=0, window_period=0, qk_norm=0, sandwich_norm=0, act="silu")
    c.update(kw)
    return c


@pytest.mark.parametrize("bad,msg", [
    (dict(head_dim=96), "head_dim"),
    (dict(hidden=100), "hidden"),
    (dict(n_head=3, n_head_kv=2), "multiple"),
    (dict(act=5), "act"),
    (dict(window=4, window_period=0), "window"),
    (dict(vocab=0), "positive"),
])
def test_config_refusals_happen_before_any_gpu_work(L, bad, msg):
    out = ctypes.c_void_p()
    rc = L.qdec_load_weights(ctypes.byref(qdec.config_struct(cfg(**bad))), None, 0, 1, 16, None, ctypes.byref(out))
    assert rc == 1
    assert msg in L.qdec_last_error().decode()
    assert out.value is None


def test_missing_and_malformed_tensors_are_refused(L):
    c = qdec.config_struct(cfg())
    out = ctypes.c_void_p()
    rc = L.qdec_load_weights(ctypes.byref(c), None, 0, 1, 16, None, ctypes.byref(out))
    assert rc == 1 and "missing" in L.qdec_last_error().decode()
    T = qdec._Tensor
    buf = (ctypes.c_uint8 * 64)()
    arr = (T * 1)(T(b"blk.0.bogus.weight", 0, 1, 16, ctypes.cast(buf, ctypes.c_void_p), 64))
    rc = L.qdec_load_weights(ctypes.byref(c), arr, 1, 1, 16, None, ctypes.byref(out))
    assert rc == 1 and "not a tensor" in L.qdec_last_error().decode()
    arr = (T * 1)(T(b"token_embd.weight", 8, 16, 64, ctypes.cast(buf, ctypes.c_void_p), 64))
    rc = L.qdec_load_weights(ctypes.byref(c), arr, 1, 1, 16, None, ctypes.byref(out))
    assert rc == 1 and "bytes" in L.qdec_last_error().decode()
    rc = L.qdec_load_weights(ctypes.byref(c), None, 0, 65, 16, None, ctypes.byref(out))
    assert rc == 1 and "max_seqs" in L.qdec_last_error().decode()


def test_null_handle_calls_are_refused(L):
    assert L.qdec_prefill(None, 0, None, 1, None, None, 0, None) == 1
    assert L.qdec_decode_step(None, None, 1, None, None, 0.0, 1.0, 0, 0, 0, None) == 1
    assert L.qdec_kv_reset(None, 0) == 1
    assert L.qdec_free(None) == 1
    assert L.qdec_poisoned(None) == -1
    out = ctypes.c_int32()
    assert L.qdec_kv_len(None, 0, ctypes.byref(out)) == 1
    assert L.qdec_debug_matmul(3, 4, 4, None, 0, None, 1, None, 0, None) == 1
    assert L.qdec_set_prefill_precision(None, 0) == 1
    assert L.qdec_debug_sample(None, 1, 1, 0.0, 1.0, 0, 0, None, None) == 1
    seqs = (ctypes.c_int32 * 1)(0)
    assert L.qdec_decode_batch(None, seqs, None, 1, None, None, 0.0, 1.0, 0, 0, 0, None) == 1
    assert L.qdec_kv_paged(None, 64, 4, None) == 1
    a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    assert L.qdec_kv_pages(None, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 1
    assert L.qdec_decode_chunks(None, ctypes.byref(a), ctypes.byref(b)) == 1
    assert L.qdec_kv_ring(None, 1, None) == 1
    assert L.qdec_kv_ring_positions(None, 0, ctypes.byref(a)) == 1
    assert L.qdec_debug_inject_fault(None, 1) == 1


def test_binding_range_checks_and_ownership():
    with pytest.raises(qdec.QdecError):
        qdec._int("seq", 2 ** 31)
    with pytest.raises(qdec.QdecError):
        qdec._int("seq", True)
    with pytest.raises(qdec.QdecError):
        qdec._int("seed", -1, qdec._U64)
    assert qdec._int("seed", 2 ** 64 - 1, qdec._U64) == 2 ** 64 - 1
    m = qdec.Model.__new__(qdec.Model)
    m._h = None
    import copy
    import pickle
    with pytest.raises(TypeError):
        copy.copy(m)
    with pytest.raises(TypeError):
        pickle.dumps(m)
    m.close()
    m.close()  # idempotent
    with pytest.raises(qdec.QdecError):
        m.kv_reset()
