"""Reference oracle for the TurboQuant KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 CPU
statement of what the compressed KV cache computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code, tables or constants with the HIP library in
``kv_cache_vector_tq_amd`` and never imports it; the product path never
imports this package.

Modules (each function cites the passage it follows; "TurboQuant on a 16GB
MacBook" is the blog post on debugging TurboQuant on an Apple M1 Pro,
"TurboQuant Family Design Study" is the CPU/WASM design study, and
"aither-kvcache" is the PyPI README of that package):

* ``codebook``   - Lloyd-Max scalar quantiser for the standard normal, scaled
                   by 1/sqrt(d), and its decision boundaries.
* ``rotation``   - dense Haar-orthogonal rotation from Gaussian draws (QR),
                   randomized Hadamard transform, QJL projection matrix.
* ``codec``      - per-vector encode (norm, rotate, quantise, pack, QJL residual
                   sketch) and dequantisation.
* ``mixed``      - mixed-channel fractional rates (2.5 and 3.5 bits): half the
                   rotated coordinates at b bits, half at b + 1.
* ``lognorm``    - u8 log-norm codes for key norms (the low-overhead mode).
* ``pages``      - fixed-size page format, FP16 recent-token ring, append.
* ``attention``  - decode attention two ways: dequantise-then-softmax (the
                   plain definition) and the compressed-domain formula.
* ``accounting`` - byte and bits-per-channel formulas.

Parity status: every function is pinned by a CPU test (``tests/test_oracle_*``)
against printed values, closed forms, brute force or invariants; none is
"parity unpinned".
"""

from . import accounting, attention, codebook, codec, lognorm, mixed, pages, rotation  # noqa: F401
