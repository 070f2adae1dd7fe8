"""Plain fp64 CPU oracle for the Gemma 4 decoder attention layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

Every function restates, in numpy float64, what the source pages say the
layer computes:

* ``norm_rope``  - plain-weight RMSNorm (QK-norm / V-norm) and rotary
  position embedding, full on sliding layers and zero-padded partial on
  global layers;
* ``attention``  - causal / sliding-window GQA softmax attention for prefill
  (a brute-force explicit-mask version for tiny inputs and a row-blocked
  band version for large ones) and single-token decode over a KV cache;
* ``kv_cache``   - KV-cache size arithmetic for the model shapes.

Parity pins (what each function is checked against, other than itself) are
listed in each module's header.  No function here is "parity unpinned".
"""

from . import norm_rope, attention, kv_cache  # noqa: F401
