"""CPU oracle for the routed MoE FFN layer on block-quantized experts.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow fp64 restatement of what the
layer computes, used to judge the HIP path. Only the test suite, the smoke check in
__graft_entry__.smoke() and the CPU-baseline leg of bench.py may import it. The
product path (the C-ABI library and its Python binding) never imports or calls it,
and shares no code, table or helper with it: the two meet only through the seeded
inputs of the `synth` package.

Modules:
  codecs  closed-form decoders of E2M1, E8M0, fp16, bf16; bf16 round-to-nearest-even;
          MXFP4 and Q8_0 block dequantization.
  moe     router logits, top-k + softmax, bucketing, expert FFN, combine, whole layer.

Every function is pinned by tests in tests/test_oracle_*.py against something other
than itself (exhaustive tables, library routines, brute force, closed-form special
cases). No function is "parity unpinned".
"""
from . import codecs, moe  # noqa: F401
