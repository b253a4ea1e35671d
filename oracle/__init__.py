"""CPU oracle for one block-diffusion denoise step (TEST INFRASTRUCTURE ONLY).

This package is the plain, slow, obviously-correct statement of what the HIP
path computes.  It is test infrastructure: only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``block_diffusion_moe_amd``) never imports, links or calls
anything here, and this package never imports the product path: the only
code the two share is the seeded input generator ``synth``.

Arithmetic: numpy in float64.  Inputs arrive as bf16 bit patterns (uint16)
and fp32 arrays and are widened exactly.  Results are rounded to bf16 only at
the two storage points the contract fixes (the SwiGLU activation and the
layer output); decisions that turn floats into integers (top-k selection,
argmax, the 0.95 commit test, the fallback pick) are taken on float32 values,
the kernels' precision, since the pages fix none.

Pages cited (title, then section):

* "Clover-35B-A3B: how a diffusion model gets to 680 tokens a second, read
  from its files" -- below "the files page".  Sections "What Clover is",
  "How it writes", "The expert selection", "What 680 tokens a second has to
  be".
* "Deep Dive -- Clover 35B: a diffusion LLM at Qwen parity, 680 tok/s" --
  below "the deep-dive page".  Section "What DiffuSpace actually shipped".

Modules:

* ``bf16``    exact bf16 <-> float conversions (round-to-nearest-even)
* ``moe``     router, top-k, SwiGLU experts, shared expert, weighted combine
* ``head``    untied head logits, mask exclusion, argmax/confidence, unmask rule
* ``norm``    RMSNorm between layers
* ``stack``   the 40-layer pre-norm residual stack
* ``brute``   dense fp64 brute force (a different algorithm) for tiny shapes
* ``counts``  the pages' parameter and byte accounting

Parity-pinning status of each function is stated in its module header.
"""
