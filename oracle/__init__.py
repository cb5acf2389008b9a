"""CPU oracle for hybrid-precision (HyQuant-style) KV attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or load
anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP path;
its only common input is the seeded generator in ``hybrid_precision_kv_amd.synth``.

Source of truth: the arXiv page "HyQuant: Hybrid-Precision Quantization for LLM
Attention" (called *the HyQuant paper* below) and the techwalker.com article
summarising it (*the techwalker article*).  Each function cites the passage it
follows.  Floating point follows the rules stated per function: quantizers run in
IEEE fp32 in a fixed operation order (so integer codes are reproducible bit for
bit), attention and scores run in fp64.

Modules:
  numerics  -- bf16 / fp16 / OCP-FP8 codecs, INT4 / INT8 / FP8 quantizers
  policy    -- anchor-count rule, vertical-line scores, top-k, the hybrid cache
               state machine (Freeze, append, refresh)
  attention -- decode attention over the hybrid cache, ReduceSoftmax merge,
               uniform-precision references, the hybrid prefill emulation

Parity status: every function is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` except the one noted "parity unpinned" below.

  * prefill P rounding (``attention.prefill_ref`` FP8/bf16 rounding of P) --
    parity unpinned: its result depends on tile order and the last ulp of exp;
    the convex-combination invariant and the exact-attention reduction are pinned,
    the rounded P codes themselves are not.
"""
