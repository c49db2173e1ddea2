"""CPU oracle for the fused-dequant Q4_K / Q5_K / Q6_K x Q8_1 matmul path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or runs this
package; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may use it.  It shares no code with the HIP path: the two
sides meet only at the byte arrays made by ``qmm_synth``.

Everything here is plain numpy.  Weights and activations are decoded to
float64 and multiplied with a float64 matmul; integer sub-block sums are
computed in int64; the Q8_1 activation quantizer is emulated step by step in
IEEE float32, since its bytes are compared bit for bit.

Pages cited (title, then section):

* [8e]  minfer ch. 06, "06 · 8e/8e② — decode MMVQ: dp4a integer dot
  products + the llama.cpp launch table".
* [MMQ] ZINC, "ZINC MMQ v2 — Fused Q4_K×Q8_1 Tensor-Core GEMM (beat
  llama.cpp)".
* [GAP] ZINC, "Prefill Gap Closure Plan — ZINC CUDA vs llama.cpp".

Readings where the pages are silent (each pinned by a test unless marked):

* Q4_K 6-bit scale/min packing: the pages call a helper whose body they do
  not print ([8e] §3.2).  Read as the public GGUF K-quant packing.
  GGUF compatibility itself is parity unpinned (no GGUF file is available);
  the packing's bijectivity and a hand-packed block are pinned.
* Q5_K layout: the pages name the format but do not give it.  Read as
  GGUF's Q5_K (the Q4_K fields plus a 32-byte plane of fifth bits); GGUF
  compatibility parity unpinned, a hand-packed block, bit bijectivity and
  the reduction to Q4_K when the fifth bits are zero pinned.
* Q6_K element -> (ql, qh) bit mapping: [8e] §3.1 says the formats follow
  GGUF semantics but prints no Q6_K code.  Read as GGUF's mapping; GGUF
  compatibility parity unpinned, bijectivity and hand-made blocks pinned.
* Q8_1 quantizer divides by ``d`` in the prose of [8e] §2 but multiplies by
  the float32 reciprocal in the code of §3.2; the code is taken.
* The Q8_1 pad bytes are written as zero.
* MoE routing weights are the raw top-k softmax probabilities; the SwiGLU
  glue between the grouped calls is silu(gate) * up (not on the pages beyond
  "swiglu producers", [8e] §3.2) -- parity unpinned beyond closed forms.
"""
from .formats import (  # noqa: F401
    q4k_fields, q4k_dequant, q5k_fields, q5k_dequant, q6k_fields, q6k_dequant, q8_1_fields, q8_1_dequant,
)
from .quantize import quantize_q8_1  # noqa: F401
from .matmul import (  # noqa: F401
    dense, abs_bound, q4k_subdots, q5k_subdots, q6k_subdots, q4k_factored, q5k_factored, q6k_factored,
)
from .moe import route_buckets, grouped, grouped_blocks, combine, swiglu  # noqa: F401
