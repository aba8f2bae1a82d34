"""CPU oracle for the W8A8 FP8 block-scaled MoE expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark use it.

The oracle is a plain, slow, obviously-correct numpy implementation of what
the expert path computes.  It shares no code, tables or constants with the
HIP path.  Floating point runs in float64 except where a quantisation decision
is made (intermediate requantisation, E8M0 exponent choice, fp8 codes): those
decisions are taken in float32, the precision the kernels take them in.

Sources (cited by page title and section; the pages are blog analyses of
FlashInfer pull requests):
  * "Blackwell W8A8 AlphaMoE expert-kernel fusion" (flashinfer PR 4287):
    section "Problem: the MoE expert bottleneck" gives the five stages
    (GEMM1 gate+up, SwiGLU, intermediate FP8 requantisation, GEMM2 down,
    combine) and the conceptual "before" kernel sequence.
  * "SM120 MoE GEMM wave+residue cost model" (flashinfer PR 4318):
    section 1 (the grouped FP8 op: a/b/scales/m_indptr, gated = gate+up),
    section 2 (the tile_m selector ladder), review notes (TileN per class).
  * "SwiGLU + MXFP8 kernel for R200 (SM107)" (flashinfer PR 8023): title and
    section 1 (gated activation to MXFP8 with 1x32 E8M0 scales, size routing).

Modules:
  formats     -- e4m3 / bf16 / E8M0 codecs, block and 1x32 MX quantisers
  route       -- stable counting sort of (token, slot) rows by expert
  moe         -- the fused-MoE reference, stage by stage (FP8 block-scaled,
                 and the MXFP8 1x32 E8M0 variant)
  gated_act   -- standalone SwiGLU + MXFP8 reference
  tile_select -- the tile_m ladder (integer logic, compared bit-exactly)
"""

from . import formats, route, moe, gated_act, tile_select  # noqa: F401
