"""Plain fp64 CPU oracle for jagged softmax attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The library (``variable_length_flash_jagged_amd``) never imports it, and this
package imports nothing from the library: the two share no code.

Sources (the pages; a citation names the page title and its section):

* "Optimizing Jagged Flash Attention with TLX" reading notes (yuxiaoba.github.io),
  sections "why unequal lengths change the problem" and "load balancing".
* "Using TLX to optimise jagged flash attention on Blackwell GPUs" (explore.n1n.ai),
  section "performance defects of padded tensors" (worked offsets example).
* "TLX Block Attention: a warp-specialized Blackwell kernel for fixed-block-sparse
  self-attention" (bittide.aicompass.dev translation), sections 2.1 (Listing 1,
  the fixed-block simplifications), 4 (backward) and 5 (scheduling).
* "Jagged Flash Attention on TLX" (aixai.ru), sections "What is Jagged Flash
  Attention", "Tile balancing and Cluster Launch Control", "dQ epilogue".

Modules:

* ``offsets``   -- offsets (cu_seqlens) arithmetic and validation.
* ``attention`` -- softmax attention forward/backward by plain definition, fp64.
* ``schedule``  -- the tile scheduler rules written out (sorted zigzag, round robin,
  contiguous divmod ranges) as the bit-exact specification of the host scheduler.
* ``block_sparse`` -- the block-sparse top-k variant (pooled query and key blocks,
  top-k key blocks per query block, attention over the kept blocks).
* ``rotary`` -- block-diagonal attention with the rotary position embedding fused in
  (rotation of q and k, and its transpose on dQ and dK).
* ``mxfp8`` -- the MXFP8 variant (OCP MX quantisation of Q, K, V; attention of the
  dequantised inputs; a bound for quantising P).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_schedule_spec.py``, ``tests/test_oracle_block_sparse.py`` and
``tests/test_oracle_rotary.py``, ``tests/test_oracle_mxfp8.py`` (worked example printed on the pages, independent
library routines, closed forms, finite differences, brute force).  Nothing here is
"parity unpinned".
"""

from .offsets import (  # noqa: F401
    offsets_from_lengths,
    lengths_from_offsets,
    validate_offsets,
    block_offsets,
)
from . import block_sparse  # noqa: F401
from . import rotary  # noqa: F401
from . import mxfp8  # noqa: F401
from .attention import (  # noqa: F401
    MODE_SELF,
    MODE_BROADCAST_Q,
    MODE_BLOCK_DIAG,
    sequence_forward,
    sequence_backward,
    attention_forward,
    attention_backward,
)
