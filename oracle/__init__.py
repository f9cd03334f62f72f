"""CPU oracle for the QLoRA linear layer and the QLoRA SwiGLU MLP block.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library (no kernels,
headers, helpers or tables); both sides only read the same seeded inputs from
``synth``.

What it computes, and from where:

* ``nf4``   - blockwise-absmax 4-bit NormalFloat quantization of a frozen base
  weight (the QLoRA format named in "LLM Fine-Tuning in 2026: Unsloth vs QLoRA
  vs Liger-Kernel", FAQ "difference between LoRA and QLoRA"; "Speed Up
  Fine-Tuning 2x with Unsloth", item 1 "4-bit Quantization"), optional
  double quantization of the absmax constants, and dequantization.  This is an
  encoding, so it is written as the sequence of steps and the GPU must match it
  bit for bit.
* ``qlora`` - the LoRA-adapted linear map h = W0 x + (alpha/r) B A x ("LLM
  Fine-Tuning in 2026", section 1) with a frozen dequantized W0, its
  hand-derived gradients with respect to x, A and B (section 2 of the same page;
  "Teaching Script FTDD-03", slide 3 "manual autograd"), and the SwiGLU MLP
  built from three such layers, with the activation recomputed from the saved
  gate/up pre-activations in the backward pass ("What is Unsloth", "Recompute
  instead of store").  These have plain definitions, so the oracle is the
  definition evaluated in float64 with no intermediate rounding.

* ``rmsnorm`` - the RMSNorm in front of the MLP block with one saved inverse
  RMS per row (the fused-RMSNorm part of section 2 of "LLM Fine-Tuning in
  2026"), forward and hand-derived backward, the definition in float64.
* ``linear_ce`` - the output head's linear projection followed by the
  cross-entropy loss, and the loss gradient with respect to the hidden states
  (section 3 of "LLM Fine-Tuning in 2026", the fused cross-entropy), the
  definition in float64.

Pins (``tests/test_oracle_*.py``) tie every function to something other than
itself: exact-rational brute force for the code search, codebook-exact blocks,
idempotence, error bounds, the B = 0 reduction to the plain base matmul, the
pages' column-vector form of the update, the merged-weight form, and central
finite differences of <Y, dY> for every gradient.
"""
from . import linear_ce, nf4, qlora, rmsnorm  # noqa: F401
