"""fp64 CPU oracle for the forward triangle multiplicative update.

TEST INFRASTRUCTURE ONLY.  The HIP library and its Python binding never import,
link or call anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` do.  The arithmetic lives in plain C
(``trimul_oracle.c``, fp64 loops); this module only compiles it with gcc and
marshals numpy arrays through ctypes.
"""
from .oracle import (build, lib_path, max_threads, trimul_full, trimul_grid, gather_grid,
                     output_stage)

__all__ = ["build", "lib_path", "max_threads", "trimul_full", "trimul_grid", "gather_grid",
           "output_stage"]
