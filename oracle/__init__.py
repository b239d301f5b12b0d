"""CPU oracle for compressed-sparse-KV decode: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation (fp64 wherever the result
is a real number) of what the decode path computes.  Only the test suite, the
package's smoke check and the bench's CPU-baseline leg may import it; the
product path never calls into it, and it shares no code, table or helper with
the HIP library.

Modules
* ``formats``  - OCP E4M3FN and E2M1 codes, the FP4 block format (E2M1 values,
  one E4M3 scale per 16 channels) and the mixed FP8/BF16 shared-KV row.
* ``decode``   - lightning-indexer scores, top-k selection, sparse attention
  over selected entries plus the sliding window (CSA), dense attention (HCA).
* ``kvbytes``  - KV-cache size accounting in closed form.
* ``tiefree``  - conditioning of seeded inputs so that the top-k set is unique
  under any fp32 evaluation order (used by tests only).

Parity status of every function is listed at the top of its module.
"""
from . import formats, decode, kvbytes, tiefree  # noqa: F401
