"""CPU oracle for the chunked gated-delta-rule (GDN) prefill forward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (``chunked_gated_delta_rule_amd``) never imports it, and this
package never imports the product: the two share no code.

Contents (each function cites the passage of the source pages it follows):

* ``recurrent``   -- fp64 token-by-token recurrence and the conv/SiLU/L2 front,
                     plain C (``gdn_oracle.c``) behind ctypes.
* ``chunked``     -- fp64 NumPy evaluation of the chunked (intra/inter) form.
* ``bruteforce``  -- exact rational arithmetic (``fractions``) on tiny inputs,
                     using the per-token transition form of the recurrence.
* ``index_table`` -- chunk-index table and its static bound, plain loops.

Pins (tests/test_oracle*.py, run with ``-m "not gpu"``): brute force on tiny
inputs, closed forms, chunk-size invariance of the chunked form, the
finite-series inverse, numpy.convolve for the front, and the page-printed
memory estimate for the static bound. No function here is "parity unpinned".
"""

from . import recurrent, chunked, bruteforce, index_table  # noqa: F401
