"""fp64 CPU oracle for packed joint text+image attention with 2D RoPE.

TEST INFRASTRUCTURE. Only the test suite, the smoke check of the package entry
file and the CPU-baseline leg of the benchmark may import or run anything in
this directory. The GPU library never calls it and shares no code with it.

Every function here is the plain definition of a step, in float64, written so
that a reader can check it against the pages by eye:

* ``packing``   -- per-sample cumulative offsets and per-token (row, col)
  positions of a packed text+image batch (Mage-Flow tech report, NR-MMDiT
  section, native-resolution packing paragraph).
* ``rope``      -- 2D rotary position embedding (mageflow.net architecture
  page, section 2, "Rotary Position Embeddings (2D RoPE)").
* ``attention`` -- joint bidirectional softmax attention restricted to each
  sample (architecture page sections 2 and 8; tech report NR-MMDiT section).
* ``rectified_flow`` -- the rectified-flow interpolation, target velocity and
  Euler / midpoint integration (architecture page, section 3).

Where the pages leave a choice open the reading taken is written in the
function's docstring.
"""
from . import attention, packing, rectified_flow, rope  # noqa: F401
