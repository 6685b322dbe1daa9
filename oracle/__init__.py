"""Plain, slow CPU oracle for the low-bit routed-MoE expert FFN.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, calls or
links this package; only the test suite, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP path: its packers,
decoders and layer arithmetic are written here, in NumPy, from the format
definitions and the method as the source pages describe it.

Sources (cited by page title and section):
  [P1] "DeepSeek-V4.1-Flash served three ways on 4xL20"
       (lcz.me/topic/2356): §1 model structure, §2 bytes-per-token arithmetic,
       §3B Strata verify law, §7 measurement discipline.
  [P3] "[Strata] DeepSeek V4.1 Flash on a single 4090" (lcz.me/post/25274):
       §二 hardware (Q8_0 dense half), §三 disk-space reconciliation,
       §五.1 per-expert mixed quantisation table, §五.3 selection-only bias.

Modules:
  formats  -- byte layouts, RTN packers (fp32 arithmetic) and exact fp64 decoders
  moe      -- router, top-k selection, softmax renormalisation, SwiGLU experts,
              weighted combine, MXFP8 activation quantiser
  sizes    -- the pages' byte arithmetic (params per expert, bytes per token,
              mixed-format averages, bandwidth ceilings)

Parity status of each function is stated in its docstring; every function is
pinned by a test in tests/test_oracle_*.py except where a docstring says
"parity unpinned".
"""

from . import formats, moe, sizes  # noqa: F401
