"""fp64 CPU oracle for TurboQuant quantization and quantized-KV decode attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The library (``attention_tq_quantize_amd``) never imports it, and this
package imports nothing from the library: the two share only the seeded input
generators of ``tq_synth``.

Everything here is the plain definition, in float64, written to be checked by
eye against the source pages. Citations name the page and its section:

  [NIK]  S. Nikolenko, "Eternal mathematics of TurboQuant: how to compress the
         KV cache down to the Shannon limit" (blog.sergeynikolenko.ru), a
         walkthrough of Zandieh et al. 2025.
  [NAH]  "What exactly TurboQuant showed" (nahornyi.ai news note).

Readings the pages leave open:
  * The codebook is stored as float32: the fp64 Lloyd-Max centroids rounded to
    nearest. "Nearest centroid" means nearest among those stored values, ties
    to the lower index.
  * sign(0) = +1 for QJL, i.e. a sign bit is 1 iff the projection is >= 0.
  * A zero vector gets norm 0, all code bits 0 and dequantizes to 0.
  * The prod residual is taken on the unit vector u = x/|x|, and the stored
    norms (|x| and |r|) are float32.
  * Bit layouts are the library's contract (vector layout and 32-vector block
    layout), re-implemented here from their written definition.

parity pins: every function below is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against closed forms, values printed on the pages,
brute force or textbook routines.
"""
from .tq_oracle import *  # noqa: F401,F403
