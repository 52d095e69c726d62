"""CPU oracle for the disentangled-attention forward (float64, numpy).

TEST INFRASTRUCTURE. This package is the slow, plainly written truth that
the HIP path is checked against. Only `tests/`, `__graft_entry__.smoke()` and
the `cpu_baseline` leg of `bench.py` may import it. It shares no code with
the HIP library (no kernels, headers, helpers or tables); the only code both
sides use is the seeded input generator in `workloads`, which holds none of
the method's arithmetic.

Modules:
  bucket    - relative-position bucket and row table, exact integers
  attention - scores, masked softmax and output per (sequence, head)
  pack      - padded <-> packed rows and their metadata
  relproj   - the per-head projections qr, kr of the relative embeddings
  backward  - gradients of the forward (and the row log-sum-exp)

Pins (tests marked "not gpu") tie the modules to things other than
themselves: exact integer identities and invariants of the bucket, a
pure-Python brute force on tiny inputs, special cases that reduce to
torch's scaled_dot_product_attention, index-revealing inputs that expose
which table row each score term reads, a hand-derived worked example
under tests/golden/, mask / packing invariants, and packing examples
worked by hand with a pure-Python brute force beside them.
"""

from . import attention, backward, bucket, pack, relproj  # noqa: F401
from .attention import (C2P, P2C, dattn_padded, dattn_rows, dattn_varlen,  # noqa: F401
                        default_scale)
from .bucket import log_bucket, rel_index_table, span  # noqa: F401
