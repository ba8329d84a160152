"""Plain, slow CPU oracle for jagged softmax attention (fp64) and its tile plan.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this package: only the test suite, the entry point's smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library.

Modules
  attention  exact attention forward/backward, evaluated per sequence and head
  planner    the host tile plan (sort by KV work, zigzag deal, the natural
             ablation plan) and the block-sparse row/column lists, as
             integer reference
  mx         the MXFP8 encoding (OCP E4M3 elements, E8M0 block scales) and
             the MXFP8 dQ pass on decoded operands

Every function states the passage it follows. All three pages used are about
the same kernel:
  [clarity]   "Meta's 3.2K-line Triton kernel outruns FlashAttention-4 on
              jagged Blackwell attention" (theclarity.today)
  [bites]     "Meta's TLX Jagged Flash Attention Beats FA4 on Blackwell With 3x
              Less Code" (ainewsbites.com)
  [radar]     "TLX porta l'attenzione jagged su Blackwell oltre FA4 con un terzo
              del codice" (ai-radar.it, English version)
"""
from . import attention, planner  # noqa: F401
