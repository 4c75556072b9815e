"""fp64 CPU oracle for the GlowQ group-shared low-rank correction path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run anything in this package.  It shares
no code with the HIP library (``rank_error_compensation_amd``), which never imports it.

  glowq_ref : inference definitions (INT4-g128 and MX dequantisation, group / solo /
              layerwise forward, W4A8, mixture of experts, the layer path with the restore
              mask, brute-force loops, the comparator)
  solve     : the offline factor solve and restore scores, used to build exact factors
              for the tiny workload and to pin the inference oracle end to end

Every function is pinned by ``tests/test_oracle_pins.py`` (checks in ``tests/pins.py``)
against closed forms, exact arithmetic, brute force, special cases or hand-worked values
(the comparator ``parity_errors`` included); none is marked "parity unpinned".
"""
from . import glowq_ref, solve  # noqa: F401
