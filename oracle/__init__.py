"""CPU oracle for the OSCAR INT2 KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, fp64 NumPy
statement of what the hot path computes, written from the pages (Together AI's
OSCAR announcement and the Qiita deployment article).  It shares no code with
the HIP library and imports nothing from it.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does.

Modules:
  rotation    calibration covariances, eigenbasis, Hadamard, bit-reversal
              permutation, composite rotations R = U H P
  quant       fp32 rotation, clipping, per-group scale/zero, INT2 codes,
              bit packing, dequantisation
  cache       the three-region per-request cache (sink / INT2 history /
              recent) and the byte format of the pool
  attention   decode attention over the dequantised cache
  accounting  bits per KV element

Parity-pin status of every function is listed in each module's docstring.
"""

from . import accounting, attention, cache, quant, rotation  # noqa: F401
