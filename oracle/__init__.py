"""CPU oracle for layer-parallel ("fuzzy") speculative decoding.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It is a plain, slow, float64 NumPy
statement of what the method computes, written from "EasySpec: Layer-Parallel
Speculative Decoding for Efficient Multi-GPU Utilization" (abstract; rebuttal
replies on Table 4, Figure 1(b), the fuzzy KV cache and bonus calibration) and
from the standard definitions those pages rely on (decoder layers, speculative
sampling).  It shares no code with the HIP path; the only inputs both sides see
come from the ``synth`` package (shapes, weights, prompts, seeds).

Modules:
  numerics  bfloat16 round-to-nearest-even helper (mirror of the bf16 path's
            rounding points)
  plan      layer-parallel set plan
  philox    Philox4x64-10 counter-based generator and the uniform streams
  model     decoder forward: sequential (precise) and layer-parallel (fuzzy)
  sampling  token sampling and the accept / resample rule
  decode    the draft -> verify -> accept -> calibrate round loop, and vanilla
            decoding
"""
