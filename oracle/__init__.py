"""CPU oracle for the NVFP4 W4A4 linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything in this package.  The
product path (the HIP library and its Python binding) never imports it and
shares no code, table or helper with it.

Modules:
  nvfp4_ref   vectorised numpy fp64 implementation (quantize, dequantize, GEMM,
              fused-scale harmonization, naive fused GEMM)
  exact       exact-rational twin written with ``fractions.Fraction`` for
              brute-force checks of ``nvfp4_ref`` on small inputs
  gdn_ref     the Gated DeltaNet recurrence, token by token in fp64 (the
              second workload: quantized projections feeding the state)

Pages cited throughout (the extracted text of five web pages on arXiv
2609.04098, "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for
the Recurrent Half of a Hybrid 27B LLM"):
  [PX]  picx.dev summary page of that title, "Introduction and Theoretical
        Foundation" > "Background", item 1 (the NVFP4 format), and
        "Gated DeltaNet Mechanics" (the log-space decay gate).
  [LIT] dmarx anthology record "LIT-800", section "Standing in the anthology"
        (NVFP4 versus MX block formats; the fused-GEMM mis-scaled gates) and
        "Key takeaways", gates bullet (the sigmoid write strength).
  [CT]  cctest.ai article "Why Gated DeltaNet Holds Up Under 4-Bit
        Quantization", "Main findings", last bullet (global-scale mismatch of
        fused GDN projections, pre-harmonized checkpoint).
  [SB]  Daily Paper Cast episode page, episode summary (the paper abstract).

Parity pins: every function in ``nvfp4_ref`` is pinned by a ``-m "not gpu"``
test (hand-worked blocks, closed forms, invariants, torch's float8 cast, the
exact twin, brute force).  The conventions below are fixed by this oracle
alone and are marked "parity unpinned" where they are defined: the sign of a
zero code, g = 1.0 for an all-zero tensor, and the choice of the first
module's scale for the naive fused GEMM.
"""
