"""GPU tests of the C ABI's failure path (tessl `python/README.md`, "Handle
ownership, closing and errors"): a HIP error in a call returns status 2 after
draining the stream and latches the handle as poisoned; later calls are
refused with status 1; the handle still frees cleanly.  The error is injected
on the host (qdec_debug_inject_fault) right after a real kernel launch, so the
drain waits on real work and no device fault occurs.  Device-resident token ids
out of range are clamped by the kernel and reported by the next call."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import decoder_gguf_quantized_amd as qdec  # noqa: E402

DEV = "cuda:0"


def tiny():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cfg = synth.get("c1")
    return cfg, synth.generate(cfg)


def err():
    return qdec.lib().qdec_last_error().decode()


def stream():
    return torch.cuda.current_stream().cuda_stream


def test_injected_fault_in_prefill():
    cfg, t = tiny()
    L = qdec.lib()
    m = qdec.Model(cfg, t, max_seqs=1, max_ctx=64)
    h = m._h
    V = cfg["vocab"]
    prompt = np.ascontiguousarray(synth.prompt(cfg), dtype=np.int32)
    logits = torch.empty(V, dtype=torch.float32, device=DEV)
    assert L.qdec_debug_inject_fault(h, 1) == 0
    rc = L.qdec_prefill(h, 0, prompt.ctypes.data, len(prompt), logits.data_ptr(), None, 0, stream())
    assert rc == 2, err()
    assert "injected" in err()
    assert L.qdec_poisoned(h) == 1
    # the failing call drained the stream before returning
    assert torch.cuda.current_stream().query()
    # every later call is refused (status 1) and names the latch
    rc = L.qdec_prefill(h, 0, prompt.ctypes.data, len(prompt), logits.data_ptr(), None, 0, stream())
    assert rc == 1 and "poisoned" in err()
    assert L.qdec_kv_reset(h, 0) == 1 and "poisoned" in err()
    assert L.qdec_debug_inject_fault(h, 0) == 1
    kv = ctypes.c_int32(-1)
    assert L.qdec_kv_len(h, 0, ctypes.byref(kv)) == 0 and kv.value == 0  # the failed call did not advance
    m.close()  # qdec_free returns 0 on a poisoned handle (close raises otherwise)
    assert m.closed


def test_injected_fault_in_decode_after_graph_capture():
    cfg, t = tiny()
    L = qdec.lib()
    V = cfg["vocab"]
    with qdec.Model(cfg, t, max_seqs=1, max_ctx=64) as m:
        prompt = synth.prompt(cfg)
        pl = torch.empty(V, dtype=torch.float32, device=DEV)
        tok = torch.empty(2, dtype=torch.int32, device=DEV)
        m.prefill(0, prompt, pl, tok[:1])
        dl = torch.empty((1, V), dtype=torch.float32, device=DEV)
        m.decode_step(tok[:1], dl, tok[1:])  # captures and replays the decode graph
        torch.cuda.synchronize()
        h = m._h
        assert L.qdec_debug_inject_fault(h, 1) == 0
        rc = L.qdec_decode_step(h, tok[1:].data_ptr(), 1, dl.data_ptr(), tok[:1].data_ptr(), 0.0, 1.0, 0, 0,
                                qdec.TOKENS_ON_DEVICE, stream())
        assert rc == 2 and "injected" in err()
        assert L.qdec_poisoned(h) == 1
        assert m.kv_len(0) == len(prompt) + 1
        assert torch.cuda.current_stream().query()
    assert m.closed


def test_injected_fault_through_the_binding():
    cfg, t = tiny()
    m = qdec.Model(cfg, t, max_seqs=1, max_ctx=64)
    pl = torch.empty(cfg["vocab"], dtype=torch.float32, device=DEV)
    m.debug_inject_fault()
    with pytest.raises(qdec.QdecPoisoned, match="injected"):
        m.prefill(0, synth.prompt(cfg), pl)
    assert m.closed  # the binding freed the poisoned handle
    with pytest.raises(qdec.QdecError, match="closed"):
        m.kv_reset()
    # a disarmed injection does nothing
    with qdec.Model(cfg, t, max_seqs=1, max_ctx=64) as m2:
        m2.debug_inject_fault()
        m2.debug_inject_fault(False)
        m2.prefill(0, synth.prompt(cfg), pl)
        torch.cuda.synchronize()


@pytest.mark.parametrize("bad", [-3, 1024, 2 ** 31 - 1])
def test_device_token_out_of_range_reports_status_2_on_the_next_call(bad):
    cfg, t = tiny()
    L = qdec.lib()
    V = cfg["vocab"]
    m = qdec.Model(cfg, t, max_seqs=1, max_ctx=64)
    h = m._h
    pl = torch.empty(V, dtype=torch.float32, device=DEV)
    m.prefill(0, synth.prompt(cfg), pl)
    tok = torch.tensor([bad], dtype=torch.int32, device=DEV)
    out = torch.empty(1, dtype=torch.int32, device=DEV)
    dl = torch.empty((1, V), dtype=torch.float32, device=DEV)
    # the step itself is enqueued (the id is only seen on the device) ...
    rc = L.qdec_decode_step(h, tok.data_ptr(), 1, dl.data_ptr(), out.data_ptr(), 0.0, 1.0, 0, 0,
                            qdec.TOKENS_ON_DEVICE, stream())
    assert rc == 0, err()
    torch.cuda.synchronize()
    # ... the kernel clamped it (the step finished with a valid token) ...
    assert 0 <= int(out.item()) < V
    assert np.isfinite(dl.cpu().numpy()).all()
    # ... and the next call reports it
    assert L.qdec_kv_reset(h, 0) == 2
    assert "outside [0, vocab)" in err()
    assert L.qdec_poisoned(h) == 1
    assert L.qdec_kv_reset(h, 0) == 1 and "poisoned" in err()
    m.close()
