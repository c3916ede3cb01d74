"""The allocation-free sampling entry point (qdec_sample_noalloc) against the
allocating one (qdec_debug_sample), through the C ABI: identical tokens on two
calls in a row, the second with a smaller input, for greedy, plain temperature
and top-p draws; and the size limits of its fixed scratch."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import decoder_gguf_quantized_amd as qdec  # noqa: E402

DEV = "cuda:0"


def run(fn, logits, temperature, top_p, seed, step):
    rows, vocab = logits.shape
    out = torch.full((rows,), -1, dtype=torch.int32, device=DEV)
    rc = fn(logits.data_ptr(), rows, vocab, ctypes.c_float(temperature), ctypes.c_float(top_p), seed, step,
            out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, qdec.lib().qdec_last_error().decode()
    return out


@pytest.mark.parametrize("temperature,top_p", [(0.0, 1.0), (1.0, 1.0), (0.7, 0.9)])
def test_noalloc_sampling_equals_the_allocating_entry_point(temperature, top_p):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = qdec.lib()
    rng = np.random.default_rng(31)
    big = torch.from_numpy((rng.standard_normal((16, 151936)) * 3).astype(np.float32)).to(DEV)
    big[3, 7] = 40.0  # a clear winner in one row
    small = torch.from_numpy((rng.standard_normal((3, 5000)) * 3).astype(np.float32)).to(DEV)
    for step, logits in enumerate((big, small)):  # second call: fewer rows, shorter rows
        got = run(L.qdec_sample_noalloc, logits, temperature, top_p, 9, step)
        want = run(L.qdec_debug_sample, logits, temperature, top_p, 9, step)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (step, got.cpu().numpy(), want.cpu().numpy())
        assert (got >= 0).all() and (got < logits.shape[1]).all()
    # the binding's wrapper takes the same path
    out = torch.empty(3, dtype=torch.int32, device=DEV)
    qdec.sample_noalloc(small, temperature, 9, 1, out, top_p=top_p)
    torch.cuda.synchronize()
    assert torch.equal(out, want)


def test_noalloc_limits_are_refused():
    L = qdec.lib()
    x = torch.zeros((65, 8), dtype=torch.float32, device=DEV)
    out = torch.empty(65, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert L.qdec_sample_noalloc(x.data_ptr(), 65, 8, 0.0, 1.0, 0, 0, out.data_ptr(), s) == 1
    assert "rows" in L.qdec_last_error().decode()
    assert L.qdec_sample_noalloc(x.data_ptr(), 1, (1 << 20) + 1, 0.0, 1.0, 0, 0, out.data_ptr(), s) == 1
    assert "vocab" in L.qdec_last_error().decode()
    assert L.qdec_sample_noalloc(None, 1, 8, 0.0, 1.0, 0, 0, out.data_ptr(), s) == 1
    assert L.qdec_sample_noalloc(x.data_ptr(), 1, 8, -1.0, 1.0, 0, 0, out.data_ptr(), s) == 1
