"""CPU float64 oracle for FP8 paged decode attention — TEST INFRASTRUCTURE.

Plain, slow, obviously-correct NumPy code that defines what the GPU library
must compute. It shares no code with the HIP path (no kernels, headers,
tables or helpers) and imports nothing from it. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does.

Source: "Smaller, faster, safer: running Kimi and GLM at scale" (Cloudflare
blog). Section "Quantizing the KV cache": the KV cache is stored as FP8 e4m3
instead of BF16, halving its size, and the attention kernel converts values
as it reads them. Section "Protecting a shared KV cache": every physical page
carries a tag that changes on reallocation, the server records the pages and
tags each request expects, the mappings are checked before decode reads, and a
mismatch aborts the affected request.

Modules:
  e4m3     OCP E4M3 decode table and round-to-nearest-even saturating encoder
  quant    amax/448 scales and quantise-on-append
  verify   per-request tag check -> abort flags
  attention  plain softmax attention over the dequantised paged cache
  combine  split partials and their log-sum-exp merge
  step     one decode step of a workload, request by request
  handoff  prefill -> decode page handoff: BF16 pages re-encoded, tags set
  int4     INT4 weight-only linear layer of the decode phase

Parity status: every function is pinned by tests/test_oracle_*.py (the step
composition by hand-worked steps in tests/golden/step_hand_worked.json); the only
unpinned quantity is the accuracy of FP8 against BF16 attention (the pages'
evidence for it is model-level benchmark scores), which is reported, never
asserted.
"""
from . import attention, combine, e4m3, handoff, int4, quant, step, verify  # noqa: F401
