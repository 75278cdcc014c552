"""CPU oracle for the streamed NF4 + LoRA training hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The
product (``memory_streamed_qlora_amd``) never imports this package and has no
CPU fallback; this package never imports the product.  The two share only the
seeded input generators in ``msq_inputs``.

Plain, slow, obviously correct: numpy in float64 for every contraction,
exact integer / fp32 arithmetic where the method fixes bits (NF4 codes, absmax,
dequantized bf16 values, dropout masks).  Every function names the passage of
the source pages it follows; where the pages are silent the docstring says
"reading:" and states the reading taken.

Source pages (cited by title and section):
  * "Poros" research post (caistrolabs.pages.dev/research/poros) -- problem
    statement, RNG state capture, the training step, memory and throughput
    paragraphs.
  * "Limitations" (caistrolabs.com/docs/limitations) -- "What 0.00e+00 means",
    "No custom kernels", "Pretraining is out of scope", "Roadmap".
  * poros-train 0.1.0 package README (PyPI metadata) -- "How it works",
    "Quickstart", "Benchmarks".
  * "Poros - Official Validation Results (NVIDIA A100 80GB PCIe)" --
    "Configuration" table, "Bitwise parity", "Benchmark matrix".

Modules: ``nf4`` (codebook, quantize, dequantize, bf16 rounding), ``philox``
(counter-based dropout masks), ``lora`` (NF4 + LoRA linear forward/backward),
``block`` (Qwen2.5-shaped decoder block forward/backward), ``step``
(embedding -> stack -> loss -> backward -> AdamW).

Parity pins: every function here is pinned by tests under ``tests/`` that
check it against closed forms, brute force, library routines or published
known-answer values.  The stack-level loss (``step``) is "parity unpinned"
against any absolute value: the pages print no loss for random weights; it is
pinned by finite differences and by its composition of pinned parts only.
"""
