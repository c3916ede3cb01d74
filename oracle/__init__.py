"""CPU oracle for the quantized decoder forward pass -- TEST INFRASTRUCTURE.

A plain, slow, float64 numpy implementation of what the GPU path computes,
written from the pages' definitions (see each module's header).  It shares no
code with the GPU library and imports nothing from it.  Only ``tests/``, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it; the product path never routes through it.

Modules:
  blocks   -- GGUF Q8_0 / Q4_0 / F32 decoding
  ops      -- RMSNorm, RoPE, attention, activations, softmax
  model    -- OracleModel: prefill / decode over a KV cache
  sampler  -- greedy argmax, Philox4x64-10, Gumbel-max temperature sampling

Pins: every function is checked in tests/test_oracle_*.py against closed
forms, invariants, brute force and independent library routines.  The one
function without a pin of its own beyond cross-checks is noted there.
"""
from . import blocks, ops, sampler  # noqa: F401
from .model import OracleModel  # noqa: F401
